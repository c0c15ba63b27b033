// Fused QKV projection + per-head RMSNorm(Q, K) + rotate-half RoPE + head-band
// store, as one gfx950 kernel.
//
// What it computes follows the pages' fused front end (docs.flashinfer.ai/api/
// comm.html, "Fused QKV Projection + Norm + RoPE + Head Exchange"; the QKV
// exchange pull request body, "Assumptions": projection -> QK-norm -> RoPE,
// fp32 norm with eps 1e-6 and one [head_dim] weight for Q and one for K, bf16
// operands and outputs), with RoPE pairing lanes i and i+64.
//
// Design (gfx950):
//  * The GEMM is computed transposed, C^T[n, m] = W[n, :] . X[m, :], with
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane owns one
//    column (here: one token) and 16 rows (here: head dims), and lanes l and
//    l+32 share the token.  A wave's 128-row n-range is exactly one head, so
//    the RMS reduction over the head is a register sum plus one exchange with
//    lane l^32, and the RoPE partners e and e+64 sit in the same lane and
//    register of n-blocks b and b+2: the whole epilogue is lane-local.
//  * Block tile 256 tokens x 256 columns (two heads), K-step 64, four waves in a
//    2 x 2 grid, each owning 128 columns (one head) x 128 tokens: 16
//    accumulators of 32x32 per wave (256 fp32 per lane).
//  * Operands are K-contiguous, read with bounds-checked buffer loads (rows
//    past M or N read as zero, so tails need no clamping), staged through a
//    double-buffered LDS ring with an XOR swizzle of the 16-byte chunks that
//    keeps both the chunk writes and the MFMA fragment reads free of bank
//    conflicts.  The next K-tile's global loads are in flight while the
//    current tile's MFMAs run.
//  * Tiles are enumerated XCD-aware: consecutive workgroups go round-robin to
//    the 8 XCDs, so each XCD is given a contiguous range of the tile order,
//    which walks groups of tile rows so that neighbouring tiles share X and W
//    panels in that XCD's L2.
#include "qkvx_internal.h"

namespace qkvx {
namespace {

constexpr int BM = 256;        // tokens per tile
constexpr int BN = 256;        // output columns per tile (two heads)
constexpr int BK = 64;         // K per pipeline stage
constexpr int NT = 256;        // threads: four waves
constexpr int GROUP_M = 8;     // tile rows walked together in the tile order
constexpr int NXCD = 8;
constexpr int CHUNKS = BK / 8;                 // 16-byte chunks per operand row
constexpr int TILE_CHUNKS = BM * CHUNKS;       // 2048 chunks per operand tile
constexpr int LOADS = TILE_CHUNKS / NT;        // 8 chunk loads per thread per operand

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Chunk position of chunk c of tile row r.  Rows are 128 bytes, so eight rows
// span 1 KB; the XOR pattern (r mod 8) ^ bit 3 of r gives every row of an
// aligned group of 8 a different 16-byte slot, and does the same for the even
// and for the odd rows of a group of 16.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    // XCD-aware remap: workgroup bid runs on XCD bid % 8; give each XCD a
    // contiguous range of the logical order.
    const int xcd = bid % NXCD;
    const int idx = bid / NXCD;
    const int per = total / NXCD;
    const int rem = total % NXCD;
    const int logical = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    // grouped order: walk group_m tile rows column by column
    const int in_group = group_m * tiles_n;
    const int g = logical / in_group;
    const int first_m = g * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int r = logical - g * in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void fused_qkv_kernel(FusedArgs a) {
    __shared__ uint4 lds_w[2 * TILE_CHUNKS];   // 2 x 32 KB
    __shared__ uint4 lds_x[2 * TILE_CHUNKS];   // 2 x 32 KB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1;      // which head of the tile
    const int wm = wave >> 1;     // which 128 tokens of the tile

    int tm, tn;
    tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int K = a.K;

    // ---- global -> LDS assignment: chunk (row = i*32 + tid/8, c = tid%8) ----
    const int lrow = tid >> 3;
    const int lc = tid & 7;
    const int wslot = lrow * CHUNKS + (lc ^ swz(lrow));    // + i * 32 * CHUNKS
    // byte sizes are below 2^32 (checked on the host); reads past them return 0
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.w, (short)0, int(uint32_t(a.N) * uint32_t(K) * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, (short)0, int(uint32_t(a.M) * uint32_t(K) * 2u), 0x00020000);
    // byte offsets of this thread's first chunk of the W and X panels
    const uint32_t gw0 = uint32_t(n0 + lrow) * uint32_t(K) * 2u + uint32_t(lc) * 16u;
    const uint32_t gx0 = uint32_t(m0 + lrow) * uint32_t(K) * 2u + uint32_t(lc) * 16u;
    const uint32_t row32 = 32u * uint32_t(K) * 2u;         // 32 rows further

    // ---- fragment reads: lane owns row (lane%32) of each 32-row block --------
    const int fr = lane & 31;
    const int hf = lane >> 5;
    int koff[4];                                            // chunk slot per K-sub-step
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[ks] = fr * CHUNKS + ((2 * ks + hf) ^ swz(fr));
    const int wbase = wn * 128 * CHUNKS;
    const int xbase = wm * 128 * CHUNKS;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 sw[LOADS], sx[LOADS];
    auto load_tile = [&](int kt) {
        const uint32_t kb = uint32_t(kt) * BK * 2u;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            sw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rw, gw0 + i * row32 + kb, 0, 0));
            sx[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rx, gx0 + i * row32 + kb, 0, 0));
        }
    };
    auto store_tile = [&](int buf) {
        uint4* lw = lds_w + buf * TILE_CHUNKS;
        uint4* lx = lds_x + buf * TILE_CHUNKS;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            lw[wslot + i * 32 * CHUNKS] = sw[i];
            lx[wslot + i * 32 * CHUNKS] = sx[i];
        }
    };

    const int KT = K / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_tile(kt + 1);
        const uint4* lw = lds_w + cur * TILE_CHUNKS + wbase;
        const uint4* lx = lds_x + cur * TILE_CHUNKS + xbase;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 af[4], bfm[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                af[b] = __builtin_bit_cast(bf16x8, lw[b * 32 * CHUNKS + koff[ks]]);
                bfm[b] = __builtin_bit_cast(bf16x8, lx[b * 32 * CHUNKS + koff[ks]]);
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[nb], bfm[mb],
                                                                         acc[nb][mb], 0, 0, 0);
        }
        if (kt + 1 < KT) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: one head (128 columns) per wave ----------------------------
    const int ncol = n0 + wn * 128;
    if (ncol >= a.N) return;
    const int p = ncol / a.hidden;                 // 0 q, 1 k, 2 v
    const int h = (ncol - p * a.hidden) >> 7;
    const int d = h / a.local_heads;
    const int j = h - d * a.local_heads;
    uint16_t* dbase = a.slot + int64_t(d) * a.region_elems + int64_t(p) * a.part_stride +
                      int64_t(j) * a.stride_h;
    const float* nw = p == 0 ? a.wq : a.wk;

#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int m = m0 + wm * 128 + mb * 32 + fr;
        if (m >= a.M) continue;
        const int bidx = m / a.s_local;
        const int s = m - bidx * a.s_local;
        const int row = a.row0 + s;                 // sequence row == position
        float v[4][16];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) v[nb][r] = acc[nb][mb][r];

        if (p < 2) {
            // RMSNorm over the head's 128 values: 64 here, 64 in lane ^ 32
            float ss = 0.f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) ss += v[nb][r] * v[nb][r];
            ss += __shfl_xor(ss, 32);
            const float inv = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
            // value (nb, r) is head dim e = 32 nb + 8 (r / 4) + 4 hf + r % 4
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 wv = *reinterpret_cast<const f32x4*>(nw + 32 * nb + 8 * g + 4 * hf);
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[nb][4 * g + q] *= inv * wv[q];
                }
            // rotate-half RoPE: dim e < 64 pairs with e + 64 (n-block nb + 2)
            const float* csr = a.cs + int64_t(row) * 128;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int e = 32 * nb + 8 * g + 4 * hf;
                    const f32x4 c = *reinterpret_cast<const f32x4*>(csr + e);
                    const f32x4 sn = *reinterpret_cast<const f32x4*>(csr + 64 + e);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float lo = v[nb][4 * g + q];
                        const float hi = v[nb + 2][4 * g + q];
                        v[nb][4 * g + q] = lo * c[q] - hi * sn[q];
                        v[nb + 2][4 * g + q] = hi * c[q] + lo * sn[q];
                    }
                }
        }
        uint16_t* orow = dbase + int64_t(bidx) * a.stride_b + int64_t(row) * a.stride_s;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int e = 32 * nb + 8 * g + 4 * hf;
                uint2 pk;
                pk.x = uint32_t(bf16_bits(v[nb][4 * g + 0])) | (uint32_t(bf16_bits(v[nb][4 * g + 1])) << 16);
                pk.y = uint32_t(bf16_bits(v[nb][4 * g + 2])) | (uint32_t(bf16_bits(v[nb][4 * g + 3])) << 16);
                *reinterpret_cast<uint2*>(orow + e) = pk;
            }
    }
}

}  // namespace

FusedPlan fused_plan() { return FusedPlan{BM, BN, BK, NT, GROUP_M}; }

hipError_t launch_fused(const FusedArgs& a_in, hipStream_t stream) {
    FusedArgs a = a_in;
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    a.group_m = GROUP_M;
    const int tiles = a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL(fused_qkv_kernel, dim3(tiles), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qkvx
