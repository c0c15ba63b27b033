// Host side of the C ABI: argument validation, sessions, receive-slot cycling
// and kernel launches.  Every check runs before anything is enqueued, so a call
// that fails leaves every buffer as it was (the pages' contract: invalid calls
// raise before any launch or collective).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>

#include "qkvx_internal.h"

using namespace qkvx;

// Compute units of the current device, cached per device (launches read it
// from any host thread).
int qkvx::device_cus() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

thread_local std::string g_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
    return status;
}

int ok() {
    g_error.clear();
    return QKVX_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(QKVX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kInt32Limit = int64_t(1) << 31;
constexpr int64_t kUint32Limit = int64_t(1) << 32;
constexpr uint16_t kPoison = 0x7FC1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [lo, hi) covered by a strided bf16 view.
struct Range {
    uintptr_t lo, hi;
};
Range view_range(const void* base, const int64_t* shape, const int64_t* stride, int dims) {
    int64_t last = 0;
    for (int i = 0; i < dims; ++i) last += (shape[i] - 1) * stride[i];
    uintptr_t lo = reinterpret_cast<uintptr_t>(base);
    return Range{lo, lo + uintptr_t(last + 1) * 2};
}
Range bytes_range(const void* base, int64_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(base);
    return Range{lo, lo + uintptr_t(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Schedule checks shared by pack and merge: counts > 0 summing to local_heads.
int check_schedule(const int* schedule, int n_chunks, int chunk, int local_heads, int* off,
                   int* count) {
    if (!schedule) return fail(QKVX_ERR_INVALID, "schedule is NULL");
    if (n_chunks < 1) return fail(QKVX_ERR_INVALID, "n_chunks must be >= 1 (got %d)", n_chunks);
    if (chunk < 0 || chunk >= n_chunks)
        return fail(QKVX_ERR_INVALID, "chunk %d outside [0, %d)", chunk, n_chunks);
    int64_t sum = 0;
    int o = 0;
    for (int i = 0; i < n_chunks; ++i) {
        if (schedule[i] <= 0)
            return fail(QKVX_ERR_DIVISIBILITY, "schedule[%d] = %d must be > 0", i, schedule[i]);
        if (i < chunk) o += schedule[i];
        sum += schedule[i];
    }
    if (sum != local_heads)
        return fail(QKVX_ERR_DIVISIBILITY, "schedule sums to %lld, local heads are %d",
                    (long long)sum, local_heads);
    *off = o;
    *count = schedule[chunk];
    return QKVX_OK;
}

int check_peers(const qkvx_peers* p, const char* name, int world, int64_t batch, int64_t s,
                int head_count, int64_t inner) {
    if (!p) return fail(QKVX_ERR_INVALID, "%s is NULL", name);
    if (p->world != world)
        return fail(QKVX_ERR_INVALID, "%s.world = %d, expected %d", name, p->world, world);
    if (p->batch < batch)
        return fail(QKVX_ERR_CAPACITY, "%s.batch = %lld < batch %lld", name, (long long)p->batch,
                    (long long)batch);
    if (p->row_offset < 0 || p->head_offset < 0)
        return fail(QKVX_ERR_INVALID, "%s offsets must be >= 0", name);
    if (p->rows < p->row_offset + s)
        return fail(QKVX_ERR_CAPACITY, "%s rows %lld < row_offset %lld + %lld", name,
                    (long long)p->rows, (long long)p->row_offset, (long long)s);
    if (p->heads < p->head_offset + head_count)
        return fail(QKVX_ERR_CAPACITY, "%s heads %lld < head_offset %lld + %d", name,
                    (long long)p->heads, (long long)p->head_offset, head_count);
    for (int i = 0; i < 3; ++i) {
        if (p->stride[i] <= 0)
            return fail(QKVX_ERR_LAYOUT, "%s.stride[%d] = %lld must be > 0", name, i,
                        (long long)p->stride[i]);
        if (p->stride[i] % 8)
            return fail(QKVX_ERR_ALIGNMENT, "%s.stride[%d] = %lld is not a multiple of 8 elements",
                        name, i, (long long)p->stride[i]);
    }
    if (p->stride[2] < inner)
        return fail(QKVX_ERR_LAYOUT, "%s.stride[2] = %lld < %lld (heads would overlap)", name,
                    (long long)p->stride[2], (long long)inner);
    const int64_t extent = (p->batch - 1) * p->stride[0] + (p->rows - 1) * p->stride[1] +
                           (p->heads - 1) * p->stride[2] + inner;
    if (extent >= kInt32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "%s spans %lld elements (limit 2^31)", name,
                    (long long)extent);
    for (int u = 0; u < world; ++u) {
        if (!p->base[u]) return fail(QKVX_ERR_INVALID, "%s.base[%d] is NULL", name, u);
        if (!aligned16(p->base[u]))
            return fail(QKVX_ERR_ALIGNMENT, "%s.base[%d] is not 16-byte aligned", name, u);
    }
    return QKVX_OK;
}

// Two peers with one base (and the shared strides) would receive into the same
// elements, so the result would depend on which store lands last.  Peers that
// are disjoint interleaved views of one tensor (different bases, overlapping
// address intervals) are legitimate and not detected here.
int check_distinct_bases(void* const* base, int world, const char* name) {
    for (int u = 0; u < world; ++u)
        for (int w = u + 1; w < world; ++w)
            if (base[u] == base[w])
                return fail(QKVX_ERR_ALIAS, "%s[%d] and %s[%d] are the same buffer", name, u, name,
                            w);
    return QKVX_OK;
}

// Byte range of the elements a call touches in peer u.
Range peers_touched(const qkvx_peers* p, int u, int64_t batch, int64_t s, int head_count,
                    int64_t inner) {
    const int64_t first = p->row_offset * p->stride[1] + p->head_offset * p->stride[2];
    const int64_t last = first + (batch - 1) * p->stride[0] + (s - 1) * p->stride[1] +
                         (head_count - 1) * p->stride[2] + inner - 1;
    uintptr_t b = reinterpret_cast<uintptr_t>(p->base[u]);
    return Range{b + uintptr_t(first) * 2, b + uintptr_t(last + 1) * 2};
}

// Session shape: the checks of qkvx_create that do not depend on the token count.
int check_shape(int hidden, int num_heads, int head_dim, int world, int layout, int rope) {
    if (head_dim != QKVX_HEAD_DIM)
        return fail(QKVX_ERR_INVALID, "head_dim must be %d (got %d)", QKVX_HEAD_DIM, head_dim);
    if (num_heads <= 0) return fail(QKVX_ERR_INVALID, "num_heads must be > 0");
    if (hidden != num_heads * head_dim)
        return fail(QKVX_ERR_INVALID, "hidden %d != num_heads %d * head_dim %d", hidden,
                    num_heads, head_dim);
    if (world < 1 || world > QKVX_MAX_WORLD)
        return fail(QKVX_ERR_INVALID, "world %d outside [1, %d]", world, QKVX_MAX_WORLD);
    if (num_heads % world)
        return fail(QKVX_ERR_DIVISIBILITY, "num_heads %d is not divisible by world %d",
                    num_heads, world);
    if (layout != QKVX_LAYOUT_BSHD && layout != QKVX_LAYOUT_FUSED)
        return fail(QKVX_ERR_LAYOUT, "layout %d is neither bshd (0) nor fused (1)", layout);
    if (rope != QKVX_ROPE_ROTATE_HALF && rope != QKVX_ROPE_INTERLEAVED)
        return fail(QKVX_ERR_INVALID, "rope %d is neither rotate-half (0) nor interleaved (1)",
                    rope);
    // W [3 hidden, hidden]: element extent below 2^31, byte offsets of padded
    // tiles below 2^32
    const int64_t w_elems = int64_t(3) * hidden * hidden;
    if (w_elems >= kInt32Limit || (int64_t(3) * hidden + 256) * hidden * 2 >= kUint32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "W_qkv [%d, %d] exceeds the 2^31-element limit",
                    3 * hidden, hidden);
    return QKVX_OK;
}

// Token capacity (max_tokens of a session, or the token count of a call without
// one): x [tokens, hidden] and one receive region of tokens * 3 * hidden
// elements stay below 2^31 elements, x's padded tiles below 2^32 bytes.
int check_tokens(int hidden, int64_t tokens, const char* name) {
    if (tokens < 1) return fail(QKVX_ERR_INVALID, "%s must be >= 1", name);
    const int64_t x_elems = tokens * hidden;
    const int64_t region = tokens * 3 * int64_t(hidden);
    if (x_elems >= kInt32Limit || (tokens + 256) * hidden * 2 >= kUint32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "%s %lld x hidden %d exceeds the 2^31 limit", name,
                    (long long)tokens, hidden);
    if (region >= kInt32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "a receive region of %lld elements exceeds 2^31",
                    (long long)region);
    return QKVX_OK;
}

}  // namespace

// ===========================================================================
// session
// ===========================================================================

struct qkvx_session {
    int hidden, heads, world, layout, rope, num_slots;
    int64_t max_tokens;
    int64_t region_elems;       // max_tokens * 3 * hidden
    uint8_t* memory;            // control area + num_slots * world regions
    uint16_t* slots;            // memory + QKVX_CTRL_BYTES
    size_t slot_bytes;          // bytes of memory
    bool owns_slots;
    bool ctrl_zero;                    // the control area is known to be zero (set by create
                                       // when it allocates, else by the first forward's clear)
    bool publish;                      // forward calls publish readiness words
    bool last_published;               // the last call did
    // device words in the control area (zero at creation)
    unsigned long long* ready;         // QKVX_MAX_WORLD readiness words
    int* timeouts;                     // wait-kernel timeout counter
    unsigned int* sched;               // kSchedWords tile-claim counters
    unsigned long long expect[QKVX_MAX_WORLD];   // word values after the last publishing call
    int64_t calls;              // successful forward calls so far
    bool has_last;
    qkvx_outputs last;
};

extern "C" {

const char* qkvx_last_error(void) { return g_error.c_str(); }

size_t qkvx_slot_bytes(int hidden, int world, int64_t max_tokens, int num_slots) {
    if (hidden <= 0 || world <= 0 || max_tokens <= 0 || num_slots <= 0) return 0;
    return size_t(QKVX_CTRL_BYTES) +
           size_t(num_slots) * size_t(world) * size_t(max_tokens) * 3u * size_t(hidden) * 2u;
}

int qkvx_create(int hidden, int num_heads, int head_dim, int world, int layout, int rope,
                int64_t max_tokens, int num_slots, void* slot_memory, size_t slot_bytes,
                qkvx_session** out) {
    if (!out) return fail(QKVX_ERR_INVALID, "out is NULL");
    *out = nullptr;
    int st = check_shape(hidden, num_heads, head_dim, world, layout, rope);
    if (st) return st;
    if (num_slots < 1) return fail(QKVX_ERR_INVALID, "num_slots must be >= 1");
    st = check_tokens(hidden, max_tokens, "max_tokens");
    if (st) return st;
    const int64_t region = max_tokens * 3 * int64_t(hidden);
    const size_t need = qkvx_slot_bytes(hidden, world, max_tokens, num_slots);
    bool owns = false;
    if (slot_memory) {
        if (slot_bytes < need)
            return fail(QKVX_ERR_CAPACITY, "slot_memory holds %zu bytes, %zu needed", slot_bytes,
                        need);
        if (reinterpret_cast<uintptr_t>(slot_memory) & 255u)
            return fail(QKVX_ERR_ALIGNMENT, "slot_memory is not 256-byte aligned");
    } else {
        // session setup: allocate, and zero the control area once (synchronously)
        hipError_t e = hipMalloc(&slot_memory, need);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc of the receive slots");
        e = hipMemset(slot_memory, 0, QKVX_CTRL_BYTES);
        if (e != hipSuccess) {
            (void)hipFree(slot_memory);      // the memset error is the one reported
            return hip_fail(e, "zeroing the session's control area");
        }
        slot_bytes = need;
        owns = true;
    }
    qkvx_session* s = new qkvx_session();
    s->hidden = hidden;
    s->heads = num_heads;
    s->world = world;
    s->layout = layout;
    s->rope = rope;
    s->num_slots = num_slots;
    s->max_tokens = max_tokens;
    s->region_elems = region;
    s->memory = static_cast<uint8_t*>(slot_memory);
    s->slots = reinterpret_cast<uint16_t*>(s->memory + QKVX_CTRL_BYTES);
    s->slot_bytes = slot_bytes;
    s->owns_slots = owns;
    s->ctrl_zero = owns;
    s->calls = 0;
    s->has_last = false;
    s->publish = false;
    s->last_published = false;
    s->ready = reinterpret_cast<unsigned long long*>(s->memory + kCtrlReady);
    s->timeouts = reinterpret_cast<int*>(s->memory + kCtrlTimeouts);
    s->sched = reinterpret_cast<unsigned int*>(s->memory + kCtrlSched);
    memset(s->expect, 0, sizeof(s->expect));
    *out = s;
    return ok();
}

int qkvx_destroy(qkvx_session* s) {
    if (!s) return fail(QKVX_ERR_INVALID, "session is NULL");
    // every allocation is released; the first failure is reported
    hipError_t first = hipSuccess;
    const char* what = nullptr;
    auto release = [&](void* p, const char* name) {
        if (!p) return;
        hipError_t e = hipFree(p);
        if (e != hipSuccess && first == hipSuccess) {
            first = e;
            what = name;
        }
    };
    if (s->owns_slots) release(s->memory, "hipFree of the receive slots");
    delete s;
    if (first != hipSuccess) return hip_fail(first, what);
    return ok();
}

// Views of one receive slot whose destination regions start region_elems
// apart at `first` (destination 0).
static void outputs_at(int heads, int world, int layout, uint16_t* first, int64_t region_elems,
                       int slot, int batch, int s_local, int rank, qkvx_outputs* o) {
    memset(o, 0, sizeof(*o));
    const int64_t hl = heads / world;
    const int64_t sg = int64_t(world) * s_local;
    o->slot = slot;
    o->world = world;
    o->layout = layout;
    o->rank = rank;
    o->batch = batch;
    o->s_global = sg;
    o->local_heads = hl;
    o->head_dim = QKVX_HEAD_DIM;
    const int64_t inner = layout == QKVX_LAYOUT_BSHD ? 128 : 384;
    o->stride[3] = 1;
    o->stride[2] = inner;
    o->stride[1] = hl * inner;
    o->stride[0] = sg * hl * inner;
    const int64_t part = layout == QKVX_LAYOUT_BSHD ? batch * sg * hl * 128 : 128;
    for (int d = 0; d < world; ++d) {
        uint16_t* base = first + int64_t(d) * region_elems;
        o->q[d] = base;
        o->k[d] = base + part;
        o->v[d] = base + 2 * part;
    }
}

static void fill_outputs(const qkvx_session* s, int slot, int batch, int s_local, int rank,
                         qkvx_outputs* o) {
    outputs_at(s->heads, s->world, s->layout,
               s->slots + int64_t(slot) * s->world * s->region_elems, s->region_elems, slot, batch,
               s_local, rank, o);
}

// The per-call checks of a forward call (session or not), all before any
// launch: pointers, token count against the capacity, rank, table, alignment,
// and no input overlapping the output memory `outputs`.
static int check_call(int hidden, int world, const void* x, int batch, int s_local,
                      const void* w_qkv, const float* q_norm_w, const float* k_norm_w,
                      const float* cos_sin, int64_t cos_sin_rows, int rank, int64_t capacity,
                      const char* capacity_name, Range outputs, const char* outputs_name) {
    if (!x || !w_qkv || !q_norm_w || !k_norm_w || !cos_sin)
        return fail(QKVX_ERR_INVALID, "x, w_qkv, q_norm_w, k_norm_w and cos_sin must be non-NULL");
    if (batch < 1 || s_local < 1)
        return fail(QKVX_ERR_INVALID, "batch %d and s_local %d must be >= 1", batch, s_local);
    const int64_t M = int64_t(batch) * s_local;
    if (M > capacity)
        return fail(QKVX_ERR_CAPACITY, "batch * s_local = %lld exceeds %s %lld", (long long)M,
                    capacity_name, (long long)capacity);
    if (rank < 0 || rank >= world)
        return fail(QKVX_ERR_INVALID, "rank %d outside [0, %d)", rank, world);
    if (cos_sin_rows < int64_t(rank + 1) * s_local)
        return fail(QKVX_ERR_CAPACITY, "cos_sin has %lld rows, positions up to %lld are needed",
                    (long long)cos_sin_rows, (long long)(int64_t(rank + 1) * s_local));
    if (cos_sin_rows * 128 >= kInt32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "cos_sin table exceeds 2^31 elements");
    if (!aligned16(x) || !aligned16(w_qkv))
        return fail(QKVX_ERR_ALIGNMENT, "x and w_qkv must start at 16-byte aligned addresses");
    if (!aligned16(q_norm_w) || !aligned16(k_norm_w) || !aligned16(cos_sin))
        return fail(QKVX_ERR_ALIGNMENT,
                    "cos_sin and the norm weights must start at 16-byte aligned addresses");
    const int64_t h = hidden;
    const Range ins[5] = {bytes_range(x, M * h * 2), bytes_range(w_qkv, 3 * h * h * 2),
                          bytes_range(q_norm_w, 512), bytes_range(k_norm_w, 512),
                          bytes_range(cos_sin, cos_sin_rows * 512)};
    const char* names[5] = {"x", "w_qkv", "q_norm_w", "k_norm_w", "cos_sin"};
    for (int i = 0; i < 5; ++i)
        if (overlap(outputs, ins[i]))
            return fail(QKVX_ERR_ALIAS, "%s overlaps %s", names[i], outputs_name);
    return QKVX_OK;
}

// Kernel arguments of one forward call writing the slot described by o.
static FusedArgs fused_args(int hidden, int heads, int world, int rope, const qkvx_outputs& o,
                            int64_t region_elems, const void* x, int batch, int s_local,
                            const void* w_qkv, const float* q_norm_w, const float* k_norm_w,
                            const float* cos_sin, int rank) {
    FusedArgs a;
    memset(&a, 0, sizeof(a));
    a.x = static_cast<const uint16_t*>(x);
    a.w = static_cast<const uint16_t*>(w_qkv);
    a.wq = q_norm_w;
    a.wk = k_norm_w;
    a.cs = cos_sin;
    a.slot = static_cast<uint16_t*>(o.q[0]);
    a.region_elems = region_elems;
    a.part_stride = static_cast<uint16_t*>(o.k[0]) - static_cast<uint16_t*>(o.q[0]);
    a.stride_b = o.stride[0];
    a.stride_s = o.stride[1];
    a.stride_h = o.stride[2];
    a.M = int32_t(int64_t(batch) * s_local);
    a.N = int32_t(3 * hidden);
    a.K = int32_t(hidden);
    a.hidden = int32_t(hidden);
    a.local_heads = heads / world;
    a.s_local = s_local;
    a.row0 = rank * s_local;
    a.rope_interleaved = rope == QKVX_ROPE_INTERLEAVED;
    a.eps = 1e-6f;
    return a;
}

int qkvx_forward(qkvx_session* s, const void* x, int batch, int s_local, const void* w_qkv,
                 const float* q_norm_w, const float* k_norm_w, const float* cos_sin,
                 int64_t cos_sin_rows, int rank, void* stream, qkvx_outputs* out) {
    if (!s) return fail(QKVX_ERR_INVALID, "session is NULL");
    int st = check_call(s->hidden, s->world, x, batch, s_local, w_qkv, q_norm_w, k_norm_w,
                        cos_sin, cos_sin_rows, rank, s->max_tokens, "max_tokens",
                        bytes_range(s->memory, int64_t(s->slot_bytes)),
                        "the session's receive slots");
    if (st) return st;
    const int64_t M = int64_t(batch) * s_local;
    const int64_t hidden = s->hidden;

    const int slot = int(s->calls % s->num_slots);
    qkvx_outputs o;
    fill_outputs(s, slot, batch, s_local, rank, &o);

    FusedArgs a = fused_args(s->hidden, s->heads, s->world, s->rope, o, s->region_elems, x, batch,
                             s_local, w_qkv, q_norm_w, k_norm_w, cos_sin, rank);
    if (s->publish) {
        a.ready = s->ready;
        const int hl = s->heads / s->world;
        a.dest_cols = (hl % 2 == 0 && hidden % 256 == 0) ? hl / 2 : 0;
        a.part_cols = int32_t(hidden / 256);
    }
    // zero from creation (or from the clear below) on: every launch leaves them zero again
    a.sched = s->sched;
    hipError_t e = hipSuccess;
    if (!s->ctrl_zero) {
        // caller-provided memory: the first call clears the control area with a
        // kernel on its own stream (no allocation, no synchronisation)
        e = launch_clear_words(reinterpret_cast<unsigned int*>(s->memory), QKVX_CTRL_BYTES / 4,
                               static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "control area clear launch");
    }
    e = launch_fused(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "fused projection launch");
    s->ctrl_zero = true;
    s->calls += 1;
    s->last_published = s->publish;
    if (s->publish) {
        const unsigned long long inc = ready_increment(M, s->heads / s->world);
        for (int d = 0; d < s->world; ++d) s->expect[d] += inc;
    }
    s->last = o;
    s->has_last = true;
    if (out) *out = o;
    return ok();
}

int qkvx_forward_noalloc(int hidden, int num_heads, int world, int layout, int rope,
                         const void* x, int batch, int s_local, const void* w_qkv,
                         const float* q_norm_w, const float* k_norm_w, const float* cos_sin,
                         int64_t cos_sin_rows, int rank, void* slot, size_t slot_bytes,
                         void* stream, qkvx_outputs* out) {
    int st = check_shape(hidden, num_heads, QKVX_HEAD_DIM, world, layout, rope);
    if (st) return st;
    if (!slot) return fail(QKVX_ERR_INVALID, "slot is NULL");
    if (batch < 1 || s_local < 1)
        return fail(QKVX_ERR_INVALID, "batch %d and s_local %d must be >= 1", batch, s_local);
    const int64_t M = int64_t(batch) * s_local;
    st = check_tokens(hidden, M, "batch * s_local");
    if (st) return st;
    const int64_t region = M * 3 * int64_t(hidden);
    const size_t need = size_t(world) * size_t(region) * 2u;
    if (slot_bytes < need)
        return fail(QKVX_ERR_CAPACITY, "slot holds %zu bytes, %zu needed", slot_bytes, need);
    if (reinterpret_cast<uintptr_t>(slot) & 255u)
        return fail(QKVX_ERR_ALIGNMENT, "slot is not 256-byte aligned");
    st = check_call(hidden, world, x, batch, s_local, w_qkv, q_norm_w, k_norm_w, cos_sin,
                    cos_sin_rows, rank, M, "batch * s_local", bytes_range(slot, int64_t(need)),
                    "slot");
    if (st) return st;
    // the current device's copy of the scratch array; its first lookup on a
    // device is the set-up step (hipGetSymbolAddress, no allocation)
    unsigned int* scratch = nullptr;
    hipError_t e = scratch_address(&scratch);
    if (e != hipSuccess) return hip_fail(e, "looking up the device scratch array");

    qkvx_outputs o;
    outputs_at(num_heads, world, layout, static_cast<uint16_t*>(slot), region, 0, batch, s_local,
               rank, &o);
    FusedArgs a = fused_args(hidden, num_heads, world, rope, o, region, x, batch, s_local, w_qkv,
                             q_norm_w, k_norm_w, cos_sin, rank);
    a.sched = scratch;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    // the tile-claim counters must start at zero: cleared by a kernel on the
    // same stream (a launch leaves them zero too, but an overlapping call on
    // the same GPU would not)
    e = launch_clear_words(scratch, kScratchWords, hs);
    if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
    e = launch_fused(a, hs);
    if (e != hipSuccess) return hip_fail(e, "fused projection launch");
    if (out) *out = o;
    return ok();
}

int qkvx_last_outputs(const qkvx_session* s, qkvx_outputs* out) {
    if (!s || !out) return fail(QKVX_ERR_INVALID, "session and out must be non-NULL");
    if (!s->has_last) return fail(QKVX_ERR_INVALID, "no call has been made on this session");
    *out = s->last;
    return ok();
}

int qkvx_poison_receive_slots(qkvx_session* s, void* stream) {
    if (!s) return fail(QKVX_ERR_INVALID, "session is NULL");
    const int64_t n = int64_t(s->num_slots) * s->world * s->region_elems;
    hipError_t e = launch_fill16(s->slots, n, kPoison, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "poison fill launch");
    return ok();
}

int qkvx_describe(const qkvx_session* s, char* buf, size_t len) {
    if (!s) return fail(QKVX_ERR_INVALID, "session is NULL");
    const FusedPlan p = fused_plan();
    char tmp[1024];
    int n = snprintf(
        tmp, sizeof(tmp),
        "{\"hidden\": %d, \"num_heads\": %d, \"head_dim\": %d, \"world\": %d, "
        "\"local_heads\": %d, \"layout\": \"%s\", \"max_tokens\": %lld, \"num_slots\": %d, "
        "\"region_elems\": %lld, \"slot_bytes\": %zu, \"owns_slots\": %s, \"calls\": %lld, "
        "\"next_slot\": %d, \"rope\": \"%s\", \"publish\": %s, \"eps\": 1e-6, "
        "\"tile\": {\"block_m\": %d, \"block_n\": %d, \"block_k\": %d, \"threads\": %d, "
        "\"group_m\": %d, \"mfma\": \"v_mfma_f32_16x16x32_bf16\", \"xcd_remap\": 8, "
        "\"order\": \"xcd_lockstep\", \"band_bytes\": %lld}}",
        s->hidden, s->heads, QKVX_HEAD_DIM, s->world, s->heads / s->world,
        s->layout == QKVX_LAYOUT_BSHD ? "bshd" : "fused", (long long)s->max_tokens,
        s->num_slots, (long long)s->region_elems, s->slot_bytes, s->owns_slots ? "true" : "false",
        (long long)s->calls, int(s->calls % s->num_slots),
        s->rope == QKVX_ROPE_INTERLEAVED ? "interleaved" : "rotate_half",
        s->publish ? "true" : "false", p.block_m, p.block_n, p.block_k,
        p.threads, p.group_m, (long long)kBandBytes);
    if (buf && len) {
        size_t c = size_t(n) < len ? size_t(n) : len - 1;
        memcpy(buf, tmp, c);
        buf[c] = 0;
    }
    g_error.clear();
    return n;
}

// ===========================================================================
// readiness words
// ===========================================================================

int qkvx_set_publish(qkvx_session* s, int enable) {
    if (!s) return fail(QKVX_ERR_INVALID, "session is NULL");
    // the words live in the session's control area: host bookkeeping only
    s->publish = enable != 0;
    return ok();
}

int qkvx_wait_word(const unsigned long long* word, unsigned long long expected, int spin_limit,
                   int* timeouts, void* stream) {
    if (!word || !timeouts) return fail(QKVX_ERR_INVALID, "word and timeouts must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(word) & 7u) || (reinterpret_cast<uintptr_t>(timeouts) & 3u))
        return fail(QKVX_ERR_ALIGNMENT, "word must be 8-byte and timeouts 4-byte aligned");
    if (spin_limit < 0) return fail(QKVX_ERR_INVALID, "spin_limit must be >= 0");
    hipError_t e = launch_wait_word(word, expected, spin_limit, timeouts,
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "wait kernel launch");
    return ok();
}

int qkvx_wait_ready(qkvx_session* s, int dest, int spin_limit, void* stream) {
    if (!s) return fail(QKVX_ERR_INVALID, "session is NULL");
    if (!s->has_last || !s->last_published)
        return fail(QKVX_ERR_INVALID, "the session's last call did not publish readiness words");
    if (dest < 0 || dest >= s->world)
        return fail(QKVX_ERR_INVALID, "dest %d outside [0, %d)", dest, s->world);
    return qkvx_wait_word(s->ready + dest, s->expect[dest], spin_limit, s->timeouts, stream);
}

int qkvx_ready_state(qkvx_session* s, unsigned long long* words, int* timeouts) {
    if (!s) return fail(QKVX_ERR_INVALID, "session is NULL");
    hipError_t e = hipSuccess;
    if (words)
        e = hipMemcpy(words, s->ready, sizeof(unsigned long long) * s->world,
                      hipMemcpyDeviceToHost);
    if (e == hipSuccess && timeouts)
        e = hipMemcpy(timeouts, s->timeouts, sizeof(int), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "reading the readiness words");
    return ok();
}

int qkvx_ready_expected(const qkvx_session* s, unsigned long long* words) {
    if (!s || !words) return fail(QKVX_ERR_INVALID, "session and words must be non-NULL");
    for (int d = 0; d < s->world; ++d) words[d] = s->expect[d];
    return ok();
}

// ===========================================================================
// head-chunk transport
// ===========================================================================

static int check_view(const qkvx_view4* v, const char* name) {
    if (!v) return fail(QKVX_ERR_INVALID, "%s is NULL", name);
    if (!v->base) return fail(QKVX_ERR_INVALID, "%s.base is NULL", name);
    for (int i = 0; i < 4; ++i)
        if (v->shape[i] < 1)
            return fail(QKVX_ERR_INVALID, "%s.shape[%d] = %lld must be >= 1", name, i,
                        (long long)v->shape[i]);
    if (v->shape[3] != QKVX_HEAD_DIM)
        return fail(QKVX_ERR_INVALID, "%s head_dim %lld != 128", name, (long long)v->shape[3]);
    if (v->stride[3] != 1)
        return fail(QKVX_ERR_LAYOUT, "%s last-dim stride %lld != 1", name, (long long)v->stride[3]);
    for (int i = 0; i < 3; ++i) {
        if (v->stride[i] <= 0)
            return fail(QKVX_ERR_LAYOUT, "%s.stride[%d] = %lld must be positive", name, i,
                        (long long)v->stride[i]);
        if (v->stride[i] % 8)
            return fail(QKVX_ERR_ALIGNMENT,
                        "%s.stride[%d] = %lld is not a multiple of 8 elements (16-byte rows)", name,
                        i, (long long)v->stride[i]);
    }
    if (!aligned16(v->base))
        return fail(QKVX_ERR_ALIGNMENT, "%s.base is not 16-byte aligned", name);
    int64_t last = 0;
    for (int i = 0; i < 4; ++i) last += (v->shape[i] - 1) * v->stride[i];
    if (last + 1 >= kInt32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "%s spans %lld elements (limit 2^31)", name,
                    (long long)(last + 1));
    return QKVX_OK;
}

int ulysses_pack_qkv_head_chunk(const qkvx_view4* q, const qkvx_view4* k, const qkvx_view4* v,
                                int world, const int* schedule, int n_chunks, int chunk,
                                const qkvx_peers* dst, void* stream) {
    const qkvx_view4* parts[3] = {q, k, v};
    const char* names[3] = {"q", "k", "v"};
    for (int i = 0; i < 3; ++i) {
        int st = check_view(parts[i], names[i]);
        if (st) return st;
    }
    for (int i = 1; i < 3; ++i)
        for (int j = 0; j < 4; ++j)
            if (parts[i]->shape[j] != q->shape[j])
                return fail(QKVX_ERR_INVALID, "%s.shape differs from q.shape", names[i]);
    if (world < 1 || world > QKVX_MAX_WORLD)
        return fail(QKVX_ERR_INVALID, "world %d outside [1, %d]", world, QKVX_MAX_WORLD);
    const int64_t B = q->shape[0], S = q->shape[1], H = q->shape[2];
    if (H % world)
        return fail(QKVX_ERR_DIVISIBILITY, "H = %lld is not divisible by world %d", (long long)H,
                    world);
    const int hl = int(H / world);
    int off = 0, hc = 0;
    int st = check_schedule(schedule, n_chunks, chunk, hl, &off, &hc);
    if (st) return st;
    st = check_peers(dst, "dst", world, B, S, hc, 3 * QKVX_HEAD_DIM);
    if (st) return st;
    st = check_distinct_bases(dst->base, world, "dst.base");
    if (st) return st;
    const int64_t total = B * S * hc * 48;
    if (total >= kInt32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "chunk payload of %lld vectors exceeds 2^31",
                    (long long)total);
    for (int u = 0; u < world; ++u) {
        Range t = peers_touched(dst, u, B, S, hc, 3 * QKVX_HEAD_DIM);
        for (int i = 0; i < 3; ++i)
            if (overlap(t, view_range(parts[i]->base, parts[i]->shape, parts[i]->stride, 4)))
                return fail(QKVX_ERR_ALIAS, "dst.base[%d] overlaps %s", u, names[i]);
    }
    PackArgs a;
    memset(&a, 0, sizeof(a));
    for (int i = 0; i < 3; ++i) {
        a.src[i] = static_cast<const uint16_t*>(parts[i]->base) + int64_t(off) * parts[i]->stride[2];
        a.sb[i] = parts[i]->stride[0];
        a.ss[i] = parts[i]->stride[1];
        a.sh[i] = parts[i]->stride[2];
    }
    a.db = dst->stride[0];
    a.ds = dst->stride[1];
    a.dh = dst->stride[2];
    a.total = uint32_t(total);
    a.local_heads = hl;
    a.div_hc = FastDiv(uint32_t(hc));
    a.div_s = FastDiv(uint32_t(S));
    {
        // bytes the three views span: the sum of their ranges, or the span of
        // their union when that is smaller (views into one tensor)
        uintptr_t lo = UINTPTR_MAX, hi = 0;
        uint64_t sum = 0;
        for (int i = 0; i < 3; ++i) {
            const Range r = view_range(parts[i]->base, parts[i]->shape, parts[i]->stride, 4);
            lo = r.lo < lo ? r.lo : lo;
            hi = r.hi > hi ? r.hi : hi;
            sum += uint64_t(r.hi - r.lo);
        }
        const uint64_t joint = uint64_t(hi - lo);
        a.source_bytes = sum < joint ? sum : joint;
    }
    for (int u = 0; u < world; ++u)
        a.dst[u] = static_cast<uint16_t*>(dst->base[u]) + dst->row_offset * dst->stride[1] +
                   dst->head_offset * dst->stride[2];
    hipError_t e = launch_pack(a, world, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pack launch");
    return ok();
}

int ulysses_merge_output_head_chunk(const qkvx_peers* src, int world, int local_heads,
                                    const int* schedule, int n_chunks, int chunk, void* out,
                                    int batch, int s_local, void* stream) {
    if (!out) return fail(QKVX_ERR_INVALID, "out is NULL");
    if (world < 1 || world > QKVX_MAX_WORLD)
        return fail(QKVX_ERR_INVALID, "world %d outside [1, %d]", world, QKVX_MAX_WORLD);
    if (local_heads < 1) return fail(QKVX_ERR_INVALID, "local_heads must be >= 1");
    if (batch < 1 || s_local < 1)
        return fail(QKVX_ERR_INVALID, "batch %d and s_local %d must be >= 1", batch, s_local);
    if (!aligned16(out)) return fail(QKVX_ERR_ALIGNMENT, "out is not 16-byte aligned");
    int off = 0, hc = 0;
    int st = check_schedule(schedule, n_chunks, chunk, local_heads, &off, &hc);
    if (st) return st;
    st = check_peers(src, "src", world, batch, s_local, hc, QKVX_HEAD_DIM);
    if (st) return st;
    const int64_t H = int64_t(world) * local_heads;
    const int64_t out_elems = int64_t(batch) * s_local * H * 128;
    if (out_elems >= kInt32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "out spans %lld elements (limit 2^31)",
                    (long long)out_elems);
    const int64_t total = int64_t(batch) * s_local * hc * 16;
    const Range orng = bytes_range(out, out_elems * 2);
    for (int u = 0; u < world; ++u)
        if (overlap(orng, peers_touched(src, u, batch, s_local, hc, QKVX_HEAD_DIM)))
            return fail(QKVX_ERR_ALIAS, "src.base[%d] overlaps out", u);
    BandCopyArgs a;
    memset(&a, 0, sizeof(a));
    a.sb = src->stride[0];
    a.ss = src->stride[1];
    a.sh = src->stride[2];
    a.db = int64_t(s_local) * H * 128;
    a.ds = H * 128;
    a.dh = 128;
    a.total = uint32_t(total);
    a.div_hc = FastDiv(uint32_t(hc));
    a.div_s = FastDiv(uint32_t(s_local));
    for (int u = 0; u < world; ++u) {
        a.src[u] = static_cast<const uint16_t*>(src->base[u]) + src->row_offset * src->stride[1] +
                   src->head_offset * src->stride[2];
        a.dst[u] = static_cast<uint16_t*>(out) + (int64_t(u) * local_heads + off) * 128;
    }
    hipError_t e = launch_band_copy(a, world, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return ok();
}

// Shared by ulysses_scatter_heads, ulysses_gather_heads and
// ulysses_pack_output_sequence_chunk: validates x and dst, then copies a
// [B, S_local, head_count] block of head vectors per peer y from
// x + y*peer_step (peer_step = H_local head strides or S_local row strides).
static int band_to_peers(const qkvx_view4* x, int world, const qkvx_peers* dst, bool split_heads,
                         void* stream, const char* what) {
    int st = check_view(x, "x");
    if (st) return st;
    if (world < 1 || world > QKVX_MAX_WORLD)
        return fail(QKVX_ERR_INVALID, "world %d outside [1, %d]", world, QKVX_MAX_WORLD);
    const int64_t B = x->shape[0];
    int64_t S, HC, step;
    if (split_heads) {
        if (x->shape[2] % world)
            return fail(QKVX_ERR_DIVISIBILITY, "H = %lld is not divisible by world %d",
                        (long long)x->shape[2], world);
        S = x->shape[1];
        HC = x->shape[2] / world;
        step = HC * x->stride[2];
    } else {
        if (x->shape[1] % world)
            return fail(QKVX_ERR_DIVISIBILITY, "S_global = %lld is not divisible by world %d",
                        (long long)x->shape[1], world);
        S = x->shape[1] / world;
        HC = x->shape[2];
        step = S * x->stride[1];
    }
    st = check_peers(dst, "dst", world, B, S, int(HC), QKVX_HEAD_DIM);
    if (st) return st;
    st = check_distinct_bases(dst->base, world, "dst.base");
    if (st) return st;
    const int64_t total = B * S * HC * 16;
    if (total >= kInt32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "%lld vectors per peer exceed 2^31", (long long)total);
    const Range xr = view_range(x->base, x->shape, x->stride, 4);
    for (int u = 0; u < world; ++u)
        if (overlap(xr, peers_touched(dst, u, B, S, int(HC), QKVX_HEAD_DIM)))
            return fail(QKVX_ERR_ALIAS, "dst.base[%d] overlaps x", u);
    BandCopyArgs a;
    memset(&a, 0, sizeof(a));
    a.sb = x->stride[0];
    a.ss = x->stride[1];
    a.sh = x->stride[2];
    a.db = dst->stride[0];
    a.ds = dst->stride[1];
    a.dh = dst->stride[2];
    a.total = uint32_t(total);
    a.div_hc = FastDiv(uint32_t(HC));
    a.div_s = FastDiv(uint32_t(S));
    for (int u = 0; u < world; ++u) {
        a.src[u] = static_cast<const uint16_t*>(x->base) + int64_t(u) * step;
        a.dst[u] = static_cast<uint16_t*>(dst->base[u]) + dst->row_offset * dst->stride[1] +
                   dst->head_offset * dst->stride[2];
    }
    hipError_t e = launch_band_copy(a, world, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, what);
    return ok();
}

int ulysses_scatter_heads(const qkvx_view4* x, int world, const qkvx_peers* dst, void* stream) {
    return band_to_peers(x, world, dst, true, stream, "scatter_heads launch");
}

int ulysses_gather_heads(const qkvx_view4* x, int world, const qkvx_peers* dst, void* stream) {
    return band_to_peers(x, world, dst, false, stream, "gather_heads launch");
}

int ulysses_pack_output_sequence_chunk(const qkvx_view4* x, int world, const qkvx_peers* dst,
                                       void* stream) {
    return band_to_peers(x, world, dst, false, stream, "output sequence pack launch");
}

int ulysses_exchange_chunks(const void* x, int world, int64_t chunk_bytes, int rank,
                            void* const* dst, void* stream) {
    if (!x) return fail(QKVX_ERR_INVALID, "x is NULL");
    if (!dst) return fail(QKVX_ERR_INVALID, "dst is NULL");
    if (world < 1 || world > QKVX_MAX_WORLD)
        return fail(QKVX_ERR_INVALID, "world %d outside [1, %d]", world, QKVX_MAX_WORLD);
    if (rank < 0 || rank >= world)
        return fail(QKVX_ERR_INVALID, "rank %d outside [0, %d)", rank, world);
    if (chunk_bytes < 1)
        return fail(QKVX_ERR_INVALID, "chunk_bytes %lld must be >= 1", (long long)chunk_bytes);
    bool vec16 = (chunk_bytes % 16) == 0 && aligned16(x);
    for (int u = 0; u < world; ++u) {
        if (!dst[u]) return fail(QKVX_ERR_INVALID, "dst[%d] is NULL", u);
        vec16 = vec16 && aligned16(dst[u]);
    }
    const int distinct = check_distinct_bases(dst, world, "dst");
    if (distinct) return distinct;
    const int64_t items = vec16 ? chunk_bytes / 16 : chunk_bytes;
    if (items >= kInt32Limit)
        return fail(QKVX_ERR_INT32_RANGE, "chunk of %lld bytes exceeds the per-peer limit",
                    (long long)chunk_bytes);
    const Range xr = bytes_range(x, chunk_bytes * world);
    for (int u = 0; u < world; ++u)
        if (overlap(xr, bytes_range(static_cast<uint8_t*>(dst[u]) + int64_t(rank) * chunk_bytes,
                                    chunk_bytes)))
            return fail(QKVX_ERR_ALIAS, "dst[%d] overlaps x", u);
    ChunkArgs a;
    memset(&a, 0, sizeof(a));
    a.src = static_cast<const uint8_t*>(x);
    a.chunk = chunk_bytes;
    for (int u = 0; u < world; ++u)
        a.dst[u] = static_cast<uint8_t*>(dst[u]) + int64_t(rank) * chunk_bytes;
    hipError_t e = launch_chunks(a, world, vec16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "exchange_chunks launch");
    return ok();
}

}  // extern "C"
