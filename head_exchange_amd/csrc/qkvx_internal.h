// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qkvx.h"

namespace qkvx {

// Unsigned 32-bit division by a runtime divisor through a multiply-high and a
// shift (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, the round-up variant):
//   l = ceil(log2 d),  m = floor(2^32 * (2^l - d) / d) + 1,
//   n / d = (mulhi(n, m) + n) >> l          for 0 <= n < 2^31, d >= 1.
// Index arithmetic of the transport kernels is bounded below 2^31, so the
// 33-bit intermediate never wraps.
struct FastDiv {
    uint32_t d;
    uint32_t m;
    uint32_t l;

    __host__ __device__ FastDiv() : d(1), m(1), l(0) {}
    __host__ explicit FastDiv(uint32_t divisor) : d(divisor) {
        uint32_t ll = 0;
        while ((uint64_t(1) << ll) < divisor) ++ll;
        l = ll;
        uint64_t mm = ((uint64_t(1) << 32) * ((uint64_t(1) << ll) - divisor)) / divisor + 1;
        m = uint32_t(mm);
    }
    __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
        uint32_t hi = __umulhi(n, m);
#else
        uint32_t hi = uint32_t((uint64_t(n) * m) >> 32);
#endif
        return (hi + n) >> l;
    }
    __host__ __device__ __forceinline__ void divmod(uint32_t n, uint32_t& q, uint32_t& r) const {
        q = div(n);
        r = n - q * d;
    }
};

// ---------------------------------------------------------------------------
// fused projection kernel: tile order and arguments
// ---------------------------------------------------------------------------

// Quotient and remainder of small non-negative integers, 0 <= a < 2^22 and
// 1 <= b < 2^22: a float product with the reciprocal (relative error a few
// units of 2^-24 on the device's approximate reciprocal, so within one of the
// exact quotient below 2^22), then one correction step each way.  The tile
// order's index arithmetic runs in one lane between two tiles while the
// workgroup's other waves wait, and the general 32-bit division sequence
// there costs about a microsecond per tile.  Every quantity it divides there
// (tile positions and counts, rows times queue indexes, columns) stays below
// 2^18: the host's limits keep tokens x hidden and 3 hidden x hidden below
// 2^31, so a launch has fewer than 2^18 tiles of 256 x 256.
__host__ __device__ __forceinline__ int div_fix(int a, int b, int q) {
    if (q * b > a) --q;
    if ((q + 1) * b <= a) ++q;
    return q;
}
__host__ __device__ __forceinline__ int small_div(int a, int b) {
#if defined(__HIP_DEVICE_COMPILE__)
    // the divisor is made opaque here, so that its reciprocal is computed at
    // each use rather than hoisted out of the kernel's loops into a register
    // held through the main loop
    int bb = b;
    asm volatile("" : "+v"(bb));
    return div_fix(a, b, int(float(a) * __builtin_amdgcn_rcpf(float(bb))));
#else
    return div_fix(a, b, int(float(a) / float(b)));
#endif
}
__host__ __device__ __forceinline__ int small_mod(int a, int b) { return a - small_div(a, b) * b; }

// The order in which a fused launch runs its tiles_m x tiles_n output tiles,
// split into nq queues (one per XCD; one for a grid that is not a multiple of
// the XCD count).  Position i < len(x) of queue x names logical tile
// logical(x, i); coords() turns a logical tile into its tile row and column.
// The tiles come in spans of tiles_m x cols tiles, run one after another: with
// readiness words (dest_cols > 0) span d holds the tiles of destination d's
// heads (dest_cols 256-column tiles in each of q, k and v, cols = 3 dest_cols),
// so that early destinations complete early; otherwise the one span is the
// whole grid.  Within a span:
//  * bands > 0 (XCD-lockstep): the tile rows are split into `bands` near-equal
//    bands, run one after another.  The queues form nq / csplit row groups of
//    csplit queues each.  In band b the rows are cut into nq / csplit
//    near-equal runs, and row group g owns run (g + b) % (nq / csplit); the
//    span's columns are cut into csplit near-equal ranges, and queue x (row
//    group x / csplit) takes range x % csplit of its group's run, walked
//    column by column.  Every queue of a column range starts a band at the
//    range's first column, so the XCDs stream the W column panels in step
//    (each comes from HBM about once per band and is then read from the MALL
//    by the others) while the band's X rows stay in the MALL.  csplit > 1
//    serves bands of few rows: the tiles an XCD runs at once then span about
//    as many rows as columns, which shares the most panels in its L2.
//  * bands == 0: groups of group_m tile rows walked column by column, shared
//    out among the queues in contiguous runs.
struct TileOrder {
    int tiles_m, tiles_n, group_m, nq;
    int bands, csplit;
    int dest_cols, part_cols;
    int cols, span, nspan, per, rem;
    int ng;                       // bands: row groups, nq / csplit
    // the queue a workgroup walks (own()): its length and, for one band in
    // one span, its row run and column range
    int own_x = -1, own_len = 0, own_r0 = 0, own_r = 0, own_c0 = 0;

    __host__ __device__ TileOrder(int tm, int tn, int gm, int queues, int nbands, int dcols,
                                  int pcols, int colsplit = 1)
        : tiles_m(tm), tiles_n(tn), group_m(gm), nq(queues), bands(nbands),
          csplit(colsplit > 0 ? colsplit : 1), dest_cols(dcols), part_cols(pcols) {
        cols = dcols > 0 ? 3 * dcols : tn;
        span = tm * cols;
        nspan = (tm * tn) / span;
        per = span / queues;
        rem = span % queues;
        ng = nq / csplit;
    }
    // bands: first tile row of band b; the run of rows queue x owns in band b
    __host__ __device__ int band_row(int b) const {
        const int n = tiles_m * b;
        return n < (1 << 22) ? small_div(n, bands) : n / bands;
    }
    __host__ __device__ int own_rows(int b, int x, int& r0) const {
        const int b0 = band_row(b), rb = band_row(b + 1) - b0;
        const int s = small_mod(small_div(x, csplit) + b, ng);
        r0 = b0 + small_div(rb * s, ng);
        return b0 + small_div(rb * (s + 1), ng) - r0;
    }
    // bands: the range of span columns queue x walks
    __host__ __device__ int own_cols(int x, int& c0) const {
        const int c = small_mod(x, csplit);
        c0 = small_div(cols * c, csplit);
        return small_div(cols * (c + 1), csplit) - c0;
    }
    // positions of queue x in one span
    __host__ __device__ int span_len(int x) const {
        if (bands > 0) {
            int rows = 0, r0, c0;
            for (int b = 0; b < bands; ++b) rows += own_rows(b, x, r0);
            return rows * own_cols(x, c0);
        }
        return per + (x < rem ? 1 : 0);
    }
    __host__ __device__ int len(int x) const {
        return x == own_x ? own_len : nspan * span_len(x);
    }
    // Keeps queue x's length and (one band, one span) its row run and column
    // range, so that its positions map to tiles with one division: a
    // workgroup's claims are almost all in its own queue, and this index
    // arithmetic runs in one lane between two tiles while the other waves wait.
    // On the device x must be the same in every lane (the workgroup's queue).
    __host__ __device__ void own(int x) {
        own_len = nspan * span_len(x);
        own_r = 0;
        if (bands == 1 && nspan == 1) {
            own_r = own_rows(0, x, own_r0);
            own_cols(x, own_c0);
        }
        own_x = x;
#if defined(__HIP_DEVICE_COMPILE__)
        // x is the same in every lane: keep the values in scalar registers
        own_len = __builtin_amdgcn_readfirstlane(own_len);
        own_r = __builtin_amdgcn_readfirstlane(own_r);
        own_r0 = __builtin_amdgcn_readfirstlane(own_r0);
        own_c0 = __builtin_amdgcn_readfirstlane(own_c0);
#endif
    }
    __host__ __device__ int logical(int x, int i) const {
        if (x == own_x && own_r > 0) {
            const int col = small_div(i, own_r);
            return (own_r0 + (i - col * own_r)) * cols + own_c0 + col;
        }
        const int ln = span_len(x);
        const int sp = nspan > 1 ? small_div(i, ln) : 0;
        i -= sp * ln;
        if (bands > 0) {
            int r0 = 0, r = 1, c0;
            const int cw = own_cols(x, c0);
            for (int b = 0; b < bands; ++b) {
                r = own_rows(b, x, r0);
                if (i < r * cw) break;
                i -= r * cw;
            }
            const int col = small_div(i, r);
            return sp * span + (r0 + (i - col * r)) * cols + c0 + col;
        }
        return sp * span + x * per + (x < rem ? x : rem) + i;
    }
    __host__ __device__ void coords(int l, int& tm, int& tn) const {
        const int sp = nspan > 1 ? small_div(l, span) : 0;
        const int rr = l - sp * span;
        int c;
        if (bands > 0) {
            tm = small_div(rr, cols);
            c = rr - tm * cols;
        } else {
            // groups of group_m rows, walked column by column
            const int in_group = group_m * cols;
            const int g = small_div(rr, in_group);
            const int first_m = g * group_m;
            const int gsize = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
            const int r = rr - g * in_group;
            c = small_div(r, gsize);
            tm = first_m + (r - c * gsize);
        }
        if (dest_cols > 0) {
            const int p = small_div(c, dest_cols);
            tn = p * part_cols + sp * dest_cols + (c - p * dest_cols);
        } else {
            tn = c;
        }
    }
};

// Bytes of X tile rows a band of the XCD-lockstep order may hold: 7/8 of the
// 256 MB MALL, the rest left to the W column panels in flight.
constexpr int64_t kBandBytes = int64_t(224) << 20;

// Bands of the XCD-lockstep order for a launch of `grid` workgroups on
// tiles_m tile rows of K-deep X panels (bm rows each), or 0 where that order
// does not apply: a grid that is not a multiple of the XCD count, or fewer
// tile rows than XCDs.
inline int lockstep_bands(int tiles_m, int K, int bm, int grid, int nxcd) {
    if (grid % nxcd != 0 || tiles_m < nxcd) return 0;
    const int64_t row_bytes = int64_t(bm) * K * 2;
    int64_t max_rows = kBandBytes / row_bytes;
    if (max_rows < nxcd) max_rows = nxcd;
    return int((tiles_m + max_rows - 1) / max_rows);
}

// Column ranges per row run of the XCD-lockstep order (TileOrder::csplit) for
// spans `cols` tile columns wide: the largest power of two, at most nxcd and
// cols, that keeps the rows an XCD owns in a band at or below the square root
// of the tiles it runs at once (grid / nxcd), so that those tiles span about
// as many rows as columns.  1 without bands.
inline int lockstep_csplit(int tiles_m, int cols, int bands, int grid, int nxcd) {
    if (bands <= 0) return 1;
    const int64_t rb = tiles_m / bands, at_once = grid / nxcd;
    int c = 1;
    while (2 * c <= nxcd && nxcd % (2 * c) == 0 && 2 * c <= cols &&
           (rb * 2 * c) * (rb * 2 * c) <= at_once * int64_t(nxcd) * nxcd)
        c *= 2;
    return c;
}

struct FusedArgs {
    const uint16_t* x;        // [M, K] bf16
    const uint16_t* w;        // [N, K] bf16
    const float* wq;          // [128]
    const float* wk;          // [128]
    const float* cs;          // [rows, 128]
    uint16_t* slot;           // region (t, 0) of the call's slot
    int64_t region_elems;     // elements between destination regions
    int64_t part_stride;      // elements between q, k and v of one destination
    int64_t stride_b, stride_s, stride_h;
    int32_t M, N, K;
    int32_t hidden;           // = K
    int32_t local_heads;      // H_local
    int32_t s_local;
    int32_t row0;             // rank * s_local: first sequence row and position
    int32_t tiles_m, tiles_n;
    int32_t group_m;          // tile-row group of the grouped tile orders
    int32_t bands;            // > 0: row bands of the XCD-lockstep order (TileOrder)
    int32_t csplit;           // column ranges per row run of that order
    int32_t rope_interleaved; // 0: pairs (i, i + 64); 1: pairs (2i, 2i + 1)
    FastDiv div_s;            // by s_local: token -> (batch, sequence row); set at launch
    float eps;
    // Readiness words (null: not published).  ready[d] grows by 2 for every
    // (m-tile, head of destination d) stored, after the stores are released
    // at agent scope; tiles then run destination by destination.
    unsigned long long* ready;
    int32_t dest_cols;        // 256-column tiles per destination and part (H_local / 2)
    int32_t part_cols;        // 256-column tiles per part (hidden / 256)
    // Tile-claim counters (null: every workgroup walks a fixed share of the
    // tiles).  Words 0-7: tiles claimed beyond the fixed ones in each queue
    // (one per XCD, or word 0 alone for a single queue); word 8: workgroups
    // finished.  Zero before a launch; the last workgroup to finish zeroes
    // them again.
    unsigned int* sched;
};

constexpr int kSchedWords = 16;   // tile-claim counter words a session keeps

// Byte offsets of a session's device words in the control area at the start of
// its slot memory (QKVX_CTRL_BYTES, zero when the session is created).
constexpr int kCtrlReady = 0;                                  // QKVX_MAX_WORLD x uint64
constexpr int kCtrlTimeouts = 8 * QKVX_MAX_WORLD;              // int
constexpr int kCtrlSched = kCtrlTimeouts + 64;                 // kSchedWords x uint32
static_assert(kCtrlSched + 4 * kSchedWords <= QKVX_CTRL_BYTES, "control area too small");
static_assert(QKVX_CTRL_BYTES % 256 == 0, "receive slots must stay 256-byte aligned");

// Readiness: a call adds this much to ready[d] of every destination d.
inline unsigned long long ready_increment(int64_t M, int local_heads) {
    return (unsigned long long)((M + 255) / 256) * 6ull * (unsigned long long)local_heads;
}

// ---------------------------------------------------------------------------
// pack / merge kernel arguments
// ---------------------------------------------------------------------------
struct PackArgs {
    const uint16_t* src[3];        // q, k, v at [0, 0, off, 0]
    int64_t sb[3], ss[3], sh[3];   // their strides (b, s, h)
    int64_t db, ds, dh;            // destination strides (b, row, head)
    uint32_t total;                // 16-byte chunks per destination
    int32_t local_heads;
    FastDiv div_hc, div_s;
    uint64_t source_bytes;         // bytes spanned by q, k and v together (launch choice)
    uint16_t* dst[QKVX_MAX_WORLD]; // peer d at [0, row_offset, head_offset, 0]
};

// A per-peer strided copy of 128-element head vectors: for peer y (< world),
// band head j (< head_count) and token (b, s) of [B, S]:
//   dst[y][b*db + s*ds + j*dh + e] = src[y][b*sb + s*ss + j*sh + e]
// Merge, whole-band scatter/gather and the output sequence split are all this
// map with different peer base pointers.
struct BandCopyArgs {
    int64_t sb, ss, sh;            // source strides (b, s, head)
    int64_t db, ds, dh;            // destination strides (b, s, head)
    uint32_t total;                // 16-byte chunks per peer: B*S*head_count*16
    FastDiv div_hc, div_s;
    const uint16_t* src[QKVX_MAX_WORLD];
    uint16_t* dst[QKVX_MAX_WORLD];
};

// Equal-length byte chunks: peer y receives bytes [y*chunk, (y+1)*chunk) of src
// at dst[y] (already offset to the sender's slot).
struct ChunkArgs {
    const uint8_t* src;
    int64_t chunk;                 // bytes per peer
    uint8_t* dst[QKVX_MAX_WORLD];
};

// The device scratch of qkvx_forward_noalloc: kScratchWords words (256 bytes)
// per GPU, of which the fused kernel's tile-claim counters use kSchedWords.
constexpr int kScratchWords = 64;
constexpr int kMaxDevices = 64;
static_assert(kSchedWords <= kScratchWords, "tile-claim counters exceed the scratch array");
// Address of the current device's copy of the scratch array (looked up once
// per device with hipGetSymbolAddress, then cached).
hipError_t scratch_address(unsigned int** out);
// One wave zeroes n words at p (a kernel, not a memset: callers may capture it).
hipError_t launch_clear_words(unsigned int* p, int n, hipStream_t stream);

// Launchers (enqueue only; arguments already validated).
hipError_t launch_fused(const FusedArgs& a, hipStream_t stream);
hipError_t launch_pack(const PackArgs& a, int world, hipStream_t stream);
hipError_t launch_band_copy(const BandCopyArgs& a, int world, hipStream_t stream);
// Compute units of the current device (cached per device).
int device_cus();
// vec16: chunk and every address are multiples of 16 bytes
hipError_t launch_chunks(const ChunkArgs& a, int world, bool vec16, hipStream_t stream);
hipError_t launch_fill16(uint16_t* p, int64_t n, uint16_t value, hipStream_t stream);
// One-wave kernel: waits until *word >= expected (agent-scope acquire), polling
// at most spin_limit times; on a timeout it adds 1 to *timeouts and returns.
hipError_t launch_wait_word(const unsigned long long* word, unsigned long long expected,
                            int spin_limit, int* timeouts, hipStream_t stream);

// Tile plan of the fused kernel (exposed for describe()).
struct FusedPlan {
    int block_m, block_n, block_k, threads, group_m;
};
FusedPlan fused_plan();

}  // namespace qkvx
