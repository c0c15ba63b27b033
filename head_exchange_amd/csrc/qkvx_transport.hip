// Transport kernels for gfx950: the head-chunk pack, the per-peer band copy
// (merge, whole-band scatter/gather, output sequence split) and the byte-chunk
// exchange.
//
// All head-vector kernels are bit copies between strided bf16 tensors whose
// innermost axis is one 128-element (256-byte) head vector, so every access is
// a 16-byte vector and a group of 16 lanes moves one whole head: a wave touches
// four 256-byte runs per instruction on each side, i.e. whole 128-byte cache
// lines.  Index maps ("Head-Chunk Layout and Transport Primitives" and "Ulysses
// Context-Parallel All-to-All" on docs.flashinfer.ai/api/comm.html):
//   pack   : dst_d[b, R0 + s, j, p*128 + e] = part_p[b, s, d*H_local + off + j, e]
//   merge  : out[b, s, u*H_local + off + j, e] = src_u[b, R0 + s, j0 + j, e]
//   scatter: dst_d[b, R0 + s, j0 + j, e] = x[b, s, d*H_local + j, e]
//   gather : dst_u[b, R0 + s, j0 + j, e] = x[b, u*S_local + s, j, e]
// The peer index (d or u) is blockIdx.y (pack with few peers) or the
// workgroup index modulo the peer count (band copies, pack with 8 or more
// peers), so the peer's base pointers are wave-uniform kernel arguments and no
// per-lane table lookup is needed; the rest of the flat 16-byte-chunk index is
// split with precomputed 32-bit dividers.
// Vectors per thread and the read cache policy of pack and the band copies are
// set by measurement (see pack_kernel and band_copy_kernel); every store is
// nontemporal.
#include "qkvx_internal.h"

namespace qkvx {
namespace {

constexpr int kThreads = 256;
// Sources of a pack at most this large (half the 256 MB MALL) are taken to be
// cache-resident and read with the default policy.
constexpr uint64_t kResidentBytes = 128ull << 20;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte vector per thread, nontemporal on both sides: the data is used
// once, so it should neither displace the caches' working set nor wait for it;
// on MI355X this form gives the highest copy rate (many short-lived waves,
// every request streaming).
__device__ __forceinline__ u32x4 load_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store_nt(uint16_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Three forms, chosen at launch (measured on the pages' schedules, back to back):
//  * RESIDENT (sources of at most kResidentBytes, fewer than 8 peers): two
//    vectors per thread from a block of 2 * kThreads consecutive vectors of
//    one peer, read with the default cache policy, so sources that still sit
//    in the 256 MB MALL are served from it (the 32-head shard's q, k, v:
//    100 MB; its schedule 44.4 -> 34.1 us).  On the larger 56-head sources
//    this form is 8 % slower than the next one;
//  * fewer than 8 peers otherwise: one vector per thread, nontemporal reads,
//    the peer is blockIdx.y; two, four or eight vectors per thread when one
//    would need more threads than the GPU holds at once and the larger count
//    would not, so that the copy runs in one dispatch wave (the two-head
//    chunks of the 56-head U4 schedule: the schedule per step 139 -> 137 us);
//  * 8 or more peers: the peer is the workgroup index modulo the peer count
//    (workgroups dispatched together read the same tokens' rows for every
//    peer), one vector per thread, nontemporal reads (48-head U8 schedule
//    236 -> 212 us; with 4 peers this form is 3-4 % slower).
// Stores are nontemporal in all three.
template <bool PEERS_ALONG_X, bool RESIDENT, int VPT>
__global__ __launch_bounds__(kThreads) void pack_kernel(PackArgs a, uint32_t world) {
    const uint32_t d = PEERS_ALONG_X ? blockIdx.x % world : blockIdx.y;
    const uint32_t c0 = (PEERS_ALONG_X ? blockIdx.x / world : blockIdx.x) * (VPT * kThreads) +
                        threadIdx.x;
    // The part's pointer and strides are picked per lane with selects on two
    // flags computed once: the compiler then loads all three parts' arguments
    // up front.  Written as an early return plus nested comparisons it emitted
    // a branch per part, each with its own scalar load and wait, which measured
    // 5 % slower on the 56-head U4 schedule.
    u32x4 v[VPT];
    uint16_t* dst[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const uint32_t c = c0 + k * kThreads;
        dst[k] = nullptr;
        if (c >= a.total) continue;
        const uint32_t e16 = c & 15u;
        uint32_t u = c >> 4;
        const uint32_t p = u % 3u;                 // q, k, v interleaved per head
        u = u / 3u;
        uint32_t tok, j, b, s;
        a.div_hc.divmod(u, tok, j);
        a.div_s.divmod(tok, b, s);
        const bool p0 = p == 0, p1 = p == 1;
        const uint16_t* src = p0 ? a.src[0] : (p1 ? a.src[1] : a.src[2]);
        const int64_t sb = p0 ? a.sb[0] : (p1 ? a.sb[1] : a.sb[2]);
        const int64_t ss = p0 ? a.ss[0] : (p1 ? a.ss[1] : a.ss[2]);
        const int64_t sh = p0 ? a.sh[0] : (p1 ? a.sh[1] : a.sh[2]);
        src += b * sb + s * ss + int64_t(d * a.local_heads + j) * sh + e16 * 8;
        dst[k] = a.dst[d] + b * a.db + s * a.ds + j * a.dh + p * 128 + e16 * 8;
        v[k] = RESIDENT ? *reinterpret_cast<const u32x4*>(src) : load_nt(src);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (dst[k]) store_nt(dst[k], v[k]);
}

// VPT vectors per thread: a workgroup copies VPT * kThreads consecutive vectors
// of one peer, all loads in flight before the stores.  Two per thread unless
// the copy would then need more threads than the GPU holds at once and four or
// eight would not (launch_band_copy): a copy that fits one dispatch wave runs
// without a second, partial wave (the two-head merge chunk of the 56-head U4
// schedule from HBM: 9.5-10.8 -> 8.1-8.8 us, level with a plain streaming copy
// of its bytes).  The peers are
// interleaved along the grid (peer = workgroup % world): workgroups dispatched
// together cover the same tokens of every peer, so a token's row of the merged
// output (or of a scatter source) is written (read) in one burst rather than in
// one pass per peer (6 % faster on the 10-head merge chunk of the 56-head U4
// schedule).  The source is read with the default cache policy: a merge's
// input is the attention output just written, and a band that stays in the
// 256 MB MALL is served from it, which nontemporal reads do not get (the
// pages' merge schedules back to back: 41.5 against 47 us on the 56-head U4
// shard, 83.5 against 96 us on the U2 shard).  From memory that no cache holds
// both policies run within 10 % of each other.  Stores stay nontemporal.
template <int VPT>
__global__ __launch_bounds__(kThreads) void band_copy_kernel(BandCopyArgs a, uint32_t world) {
    const uint32_t y = blockIdx.x % world;
    const uint32_t c0 = (blockIdx.x / world) * (VPT * kThreads) + threadIdx.x;
    u32x4 v[VPT];
    uint16_t* dst[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const uint32_t c = c0 + k * kThreads;
        dst[k] = nullptr;
        if (c >= a.total) continue;
        const uint32_t e16 = c & 15u;
        uint32_t tok, j, b, s;
        a.div_hc.divmod(c >> 4, tok, j);
        a.div_s.divmod(tok, b, s);
        dst[k] = a.dst[y] + b * a.db + s * a.ds + j * a.dh + e16 * 8;
        v[k] = *reinterpret_cast<const u32x4*>(a.src[y] + b * a.sb + s * a.ss + j * a.sh + e16 * 8);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (dst[k]) store_nt(dst[k], v[k]);
}

// Byte chunks, 16 bytes per thread (chunk and addresses 16-byte aligned).
__global__ __launch_bounds__(kThreads) void chunk16_kernel(ChunkArgs a) {
    const uint32_t y = blockIdx.y;
    const int64_t i = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * 16;
    if (i >= a.chunk) return;
    const u32x4 v = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(a.src + int64_t(y) * a.chunk + i));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.dst[y] + i));
}

// Byte chunks of any length and alignment, one byte per thread.
__global__ __launch_bounds__(kThreads) void chunk1_kernel(ChunkArgs a) {
    const uint32_t y = blockIdx.y;
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= a.chunk) return;
    a.dst[y][i] = a.src[int64_t(y) * a.chunk + i];
}

__global__ __launch_bounds__(kThreads) void fill16_kernel(uint16_t* p, int64_t n, uint32_t pattern) {
    const int64_t nvec = n / 8;
    const uint4 v = make_uint4(pattern, pattern, pattern, pattern);
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nvec; i += stride)
        reinterpret_cast<uint4*>(p)[i] = v;
    // tail (fewer than 8 elements), written by the first lanes of block 0
    if (blockIdx.x == 0 && threadIdx.x < n - nvec * 8)
        p[nvec * 8 + threadIdx.x] = uint16_t(pattern);
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, int world, hipStream_t stream) {
    if (a.total == 0) return hipSuccess;
    const uint32_t w = uint32_t(world);
    const uint64_t resident = uint64_t(device_cus()) * 2048u, vectors = uint64_t(a.total) * w;
    if (world >= 8) {
        const uint32_t blocks = (a.total + kThreads - 1) / kThreads;            // per peer
        hipLaunchKernelGGL((pack_kernel<true, false, 1>), dim3(blocks * w), dim3(kThreads), 0,
                           stream, a, w);
    } else if (a.source_bytes <= kResidentBytes) {
        const uint32_t blocks = (a.total + 2 * kThreads - 1) / (2 * kThreads);  // per peer
        hipLaunchKernelGGL((pack_kernel<false, true, 2>), dim3(blocks, w), dim3(kThreads), 0,
                           stream, a, w);
    } else if (vectors > resident && vectors <= 8 * resident) {
        const int vpt = vectors <= 2 * resident ? 2 : vectors <= 4 * resident ? 4 : 8;
        const uint32_t blocks = (a.total + vpt * kThreads - 1) / (vpt * kThreads);  // per peer
        if (vpt == 2)
            hipLaunchKernelGGL((pack_kernel<false, false, 2>), dim3(blocks, w), dim3(kThreads), 0,
                               stream, a, w);
        else if (vpt == 4)
            hipLaunchKernelGGL((pack_kernel<false, false, 4>), dim3(blocks, w), dim3(kThreads), 0,
                               stream, a, w);
        else
            hipLaunchKernelGGL((pack_kernel<false, false, 8>), dim3(blocks, w), dim3(kThreads), 0,
                               stream, a, w);
    } else {
        const uint32_t blocks = (a.total + kThreads - 1) / kThreads;            // per peer
        hipLaunchKernelGGL((pack_kernel<false, false, 1>), dim3(blocks, w), dim3(kThreads), 0,
                           stream, a, w);
    }
    return hipGetLastError();
}

hipError_t launch_band_copy(const BandCopyArgs& a, int world, hipStream_t stream) {
    if (a.total == 0) return hipSuccess;
    const uint32_t w = uint32_t(world);
    // threads the GPU holds at once (2048 per compute unit)
    const uint64_t resident = uint64_t(device_cus()) * 2048u, vectors = uint64_t(a.total) * w;
    int vpt = 2;
    if (vectors > 2 * resident) {
        if (vectors <= 4 * resident) vpt = 4;
        else if (vectors <= 8 * resident) vpt = 8;
    }
    dim3 grid(((a.total + vpt * kThreads - 1) / (vpt * kThreads)) * w);
    if (vpt == 8)
        hipLaunchKernelGGL(band_copy_kernel<8>, grid, dim3(kThreads), 0, stream, a, w);
    else if (vpt == 4)
        hipLaunchKernelGGL(band_copy_kernel<4>, grid, dim3(kThreads), 0, stream, a, w);
    else
        hipLaunchKernelGGL(band_copy_kernel<2>, grid, dim3(kThreads), 0, stream, a, w);
    return hipGetLastError();
}

hipError_t launch_chunks(const ChunkArgs& a, int world, bool vec16, hipStream_t stream) {
    if (a.chunk == 0) return hipSuccess;
    const int64_t per_thread = vec16 ? 16 : 1;
    const int64_t items = (a.chunk + per_thread - 1) / per_thread;
    dim3 grid(uint32_t((items + kThreads - 1) / kThreads), world);
    if (vec16)
        hipLaunchKernelGGL(chunk16_kernel, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(chunk1_kernel, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fill16(uint16_t* p, int64_t n, uint16_t value, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const uint32_t pattern = uint32_t(value) | (uint32_t(value) << 16);
    int64_t blocks = (n / 8 + kThreads - 1) / kThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill16_kernel, dim3(uint32_t(blocks)), dim3(kThreads), 0, stream, p, n,
                       pattern);
    return hipGetLastError();
}

}  // namespace qkvx
