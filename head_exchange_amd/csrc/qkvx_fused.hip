// Fused QKV projection + per-head RMSNorm(Q, K) + rotate-half RoPE + head-band
// store, as one gfx950 kernel.
//
// What it computes follows the pages' fused front end (docs.flashinfer.ai/api/
// comm.html, "Fused QKV Projection + Norm + RoPE + Head Exchange"; the QKV
// exchange pull request body, "Assumptions": projection -> QK-norm -> RoPE,
// fp32 norm with eps 1e-6 and one [head_dim] weight for Q and one for K, bf16
// operands and outputs), with RoPE pairing lanes i and i+64 (rotate-half) or,
// as in the pages' operator, lanes 2i and 2i+1 (interleaved).
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
//  * Persistent: one workgroup per CU walks its share of the tiles, and the
//    K-tiles of consecutive output tiles form one continuous load stream, so
//    the next tile's first K-tiles are in flight while the current tile's
//    epilogue runs.  In each round the 8 XCDs (workgroup b runs on XCD b % 8)
//    take consecutive ranges of a tile order that walks groups of tile rows
//    column by column, so the tiles an XCD runs together share X and W
//    panels in its L2.
#include "qkvx_internal.h"

namespace qkvx {
namespace {

constexpr int BM = 256;        // tokens per tile
constexpr int BN = 256;        // output columns per tile (two heads)
constexpr int BK = 64;         // K per LDS stage (128 bytes of each operand row)
constexpr int NT = 256;        // threads: four waves
constexpr int GROUP_M = 8;     // tile rows walked together in the tile order
constexpr int NXCD = 8;
constexpr int CHUNKS = BK / 8;                 // 16-byte chunks per operand row
// LDS image of one operand stage: 32 blocks of 8 rows x 128 bytes, each block
// followed by 16 bytes of padding (65 chunks per block).
constexpr int BLOCK_CHUNKS = 65;
constexpr int STAGE_CHUNKS = 32 * BLOCK_CHUNKS;   // 2080 chunks = 33280 bytes
constexpr int LOADS = 32 / 4;                  // block loads per wave per operand per stage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// LDS chunk index of chunk c of tile row r of one operand stage: block r / 8
// holds rows 8 (r / 8) .. + 7 as 128 contiguous bytes each, and every 1 KB block
// is followed by 16 bytes of padding.  A direct load (64 lanes x 16 bytes into
// 1 KB of LDS) therefore reads eight consecutive rows' 128-byte segments in
// ascending order -- one 128-byte request each.
__device__ __forceinline__ int lds_chunk(int r, int c) {
    return (r >> 3) * BLOCK_CHUNKS + (r & 7) * CHUNKS + c;
}

// Row of a 128-row wave range that MFMA row i (0..31) of 32-row block nb maps
// to.  Lanes i..i+7 read the same chunk of rows 8 apart, i.e. of eight
// consecutive blocks 1040 bytes apart: distinct LDS banks (32 and 64 banks).
__device__ __forceinline__ int mfma_row(int nb, int i) {
    return 64 * (nb >> 1) + 8 * (i & 7) + 4 * (nb & 1) + (i >> 3);
}

// Tile coordinates of logical tile l: groups of group_m tile rows, walked
// column by column.
__device__ __forceinline__ void tile_coords(int l, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
    const int in_group = group_m * tiles_n;
    const int g = l / in_group;
    const int first_m = g * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int r = l - g * in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void fused_qkv_kernel(FusedArgs a) {
    // Two LDS stages per operand, as separate objects so that the compiler can
    // tell a direct load into one stage from fragment reads of the other.
    __shared__ uint4 lw0[STAGE_CHUNKS], lw1[STAGE_CHUNKS];   // 33280 bytes each
    __shared__ uint4 lx0[STAGE_CHUNKS], lx1[STAGE_CHUNKS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wn = wave & 1;      // which head of the tile
    const int wm = wave >> 1;     // which 128 tokens of the tile

    // ---- tile schedule ---------------------------------------------------------
    // XCD x (workgroups b with b % 8 == x) owns a contiguous eighth of the
    // logical tile order; its G/8 workgroups walk that range G/8 tiles at a
    // time, so the 8 XCDs sweep the W panels at the same pace (sharing them
    // through the last-level cache) while each XCD's concurrent tiles share
    // panels in its L2.
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int total = a.tiles_m * a.tiles_n;
    int first, stride, end;
    if (G % NXCD == 0) {
        const int x = bid % NXCD;
        const int per = total / NXCD, rem = total % NXCD;
        first = x * per + min(x, rem) + bid / NXCD;
        end = (x + 1) * per + min(x + 1, rem);
        stride = G / NXCD;
    } else {
        first = bid;
        end = total;
        stride = G;
    }
    if (first >= end) return;
    const int K = a.K;
    auto tile_origin = [&](int l, int& m0, int& n0) {
        int tm, tn;
        tile_coords(l, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
        m0 = tm * BM;
        n0 = tn * BN;
    };

    // ---- global -> LDS: direct loads (buffer_load ... lds) ----------------------
    // Instruction i of wave w fills block b = 4 i + w of a stage: lane L brings
    // chunk L % 8 of tile row 8 b + L / 8 to LDS offset 16 L of the block.
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.w, (short)0, int(uint32_t(a.N) * uint32_t(K) * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, (short)0, int(uint32_t(a.M) * uint32_t(K) * 2u), 0x00020000);
    // byte sizes are below 2^32 (checked on the host); reads past them return 0
    const uint32_t rowbytes = uint32_t(K) * 2u;
    const int wv = wave;
    const uint32_t lrow = uint32_t(8 * wv + (lane >> 3));
    // this lane's byte offset of K-tile 0 of a tile's W panel (origin n0) or X
    // panel (origin m0)
    auto panel_offset = [&](int origin) {
        return (uint32_t(origin) + lrow) * rowbytes + uint32_t(lane & 7) * 16u;
    };

    // ---- fragment reads: lane i%32 owns MFMA row i%32 of each 32-row block ----
    const int fr = lane & 31;
    const int hf = lane >> 5;
    int woff[4], xoff[4];                                   // chunk index of row, chunk hf
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        woff[b] = lds_chunk(wn * 128 + mfma_row(b, fr), hf);
        xoff[b] = lds_chunk(wm * 128 + mfma_row(b, fr), hf);
    }

    f32x16 acc[4][4];

    // Request K-tile kt of the panels at (gw0, gx0) into stage s: 2 x LOADS
    // block loads per wave.
    auto load_stage = [&](uint32_t gw0, uint32_t gx0, int kt, int s) {
        const uint32_t kb = uint32_t(kt) * BK * 2u;
        typedef __attribute__((address_space(3))) uint4 lds_uint4;
        lds_uint4* dw = (lds_uint4*)((s ? lw1 : lw0) + wv * BLOCK_CHUNKS);
        lds_uint4* dx = (lds_uint4*)((s ? lx1 : lx0) + wv * BLOCK_CHUNKS);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const uint32_t roff = uint32_t(32 * i) * rowbytes + kb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(dw + 4 * i * BLOCK_CHUNKS), 16,
                gw0 + roff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)(dx + 4 * i * BLOCK_CHUNKS), 16,
                gx0 + roff, 0, 0, 0);
        }
    };

    // Fragments of one 16-K sub-step: four 32-row blocks of W (A operand) and of
    // X (B operand); sub-step ks reads chunks 2 ks + hf.  Two sets, A and B.
    bf16x8 fa_a[4], fb_a[4], fa_b[4], fb_b[4];
    auto read_frags = [&](int s, int ks, bf16x8* fa, bf16x8* fb) {
        const uint4* w = s ? lw1 : lw0;
        const uint4* x = s ? lx1 : lx0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            fa[b] = __builtin_bit_cast(bf16x8, w[woff[b] + 2 * ks]);
            fb[b] = __builtin_bit_cast(bf16x8, x[xoff[b] + 2 * ks]);
        }
    };
    auto mfmas = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[nb], fb[mb], acc[nb][mb],
                                                                     0, 0, 0);
    };

    // ---- main loop ------------------------------------------------------------
    // The K-tiles of this workgroup's output tiles form one stream.  The code
    // between two workgroup barriers (one scheduling region) handles K-tile kt
    // in stage s = kt % 2:
    //   the sub-step-3 MFMAs of K-tile kt-1 (its fragments are in set B);
    //   the loads of K-tile kt+1 into the other stage (free since the barrier),
    //   one instruction per two MFMAs over the first half of the region, so
    //   that the address unit never fills up and stalls the wave's in-order
    //   MFMA issue, while the last load still has half a region to arrive;
    //   the fragment reads of K-tile kt's four sub-steps and the MFMAs of its
    //   sub-steps 0..2, each sub-step's reads overlapping the previous MFMAs;
    // then a wait for this wave's loads and LDS reads, and the barrier.
    // sched_group_barrier pins the interleaving (0x008 MFMA, 0x020 VMEM read,
    // 0x100 DS read).
    const int KT = K / BK;                                  // = 2 * heads: even
    // Panels of the current tile and of this workgroup's next tile; past its
    // last tile the "next" requests re-read the current tile (in bounds, unused).
    int m0, n0, m0_next, n0_next;
    tile_origin(first, m0, n0);
    int next = first + stride;
    tile_origin(next < end ? next : first, m0_next, n0_next);
    uint32_t gw_cur = panel_offset(n0), gx_cur = panel_offset(m0);
    uint32_t gw_nxt = panel_offset(n0_next), gx_nxt = panel_offset(m0_next);
    // load K-tile index kidx of the stream (kidx >= KT: the next output tile)
    auto load_k = [&](int kidx, int stage) {
        const bool nx = kidx >= KT;
        load_stage(nx ? gw_nxt : gw_cur, nx ? gx_nxt : gx_cur, nx ? kidx - KT : kidx, stage);
    };

    // Region of K-tile kt (stage s); `steady` adds the previous K-tile's
    // sub-step-3 MFMAs and the loads of K-tile kt + 1.
    auto region = [&](int kt, int s, bool steady) {
        if (steady) {
            mfmas(fa_b, fb_b);
            load_k(kt + 1, s ^ 1);
        }
        read_frags(s, 0, fa_a, fb_a);
        read_frags(s, 1, fa_b, fb_b);
        mfmas(fa_a, fb_a);
        read_frags(s, 2, fa_a, fb_a);
        mfmas(fa_b, fb_b);
        read_frags(s, 3, fa_b, fb_b);
        mfmas(fa_a, fb_a);
        if (steady) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
        } else {
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        }
#pragma unroll
        for (int i = 0; i < (steady ? 16 : 24); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // ---- epilogue: one head (128 columns) per wave ----------------------------
    // Accumulator register reg of n-block nb in lane-half hf holds head dim
    //   e = 64 (nb / 2) + 32 hf + 8 (reg % 4) + 4 (nb % 2) + reg / 4
    // of the token of MFMA column fr of m-block mb, tile token
    //   wm * 128 + mfma_row(mb, fr).
    // Registers q, q+4, q+8, q+12 hold four consecutive dims; n-blocks 2h and
    // 2h+1 continue each other (16 bytes of bf16); n-block nb+2 holds e + 64.
  auto epilogue = [&](int m0, int n0) {
    const int ncol = n0 + wn * 128;
    if (ncol >= a.N) return;
    const int p = ncol / a.hidden;                 // 0 q, 1 k, 2 v
    const int h = (ncol - p * a.hidden) >> 7;
    const int d = h / a.local_heads;
    const int j = h - d * a.local_heads;
    uint16_t* dbase = a.slot + int64_t(d) * a.region_elems + int64_t(p) * a.part_stride +
                      int64_t(j) * a.stride_h;
    const bool qk = p < 2;
    const float* nw = p == 0 ? a.wq : a.wk;

#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        // tokens past M (ragged last tile) are computed on token M - 1 and not stored
        const int m_tile = m0 + wm * 128 + mfma_row(mb, fr);
        const bool in_range = m_tile < a.M;
        const int m = in_range ? m_tile : a.M - 1;
        const int bidx = m / a.s_local;
        const int s = m - bidx * a.s_local;
        const int row = a.row0 + s;                 // sequence row == position
        // Accumulators are read out of AGPRs one m-block at a time; written as
        // explicit reads so that the compiler does not copy all 256 of them into
        // VGPRs at the loop exit (which would spill).
        float v[4][16];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[nb][r]) : "a"(acc[nb][mb][r]));

        if (qk) {
            // RMSNorm over the head's 128 values: 64 here, 64 in lane ^ 32
            float ss = 0.f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) ss += v[nb][r] * v[nb][r];
            ss += __shfl_xor(ss, 32);
            const float inv = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
            const float* csr = a.cs + int64_t(row) * 128;
            if (a.rope_interleaved) {
                // pairs (2i, 2i+1): registers q + 4 g hold dims E + g, E = e(nb, q), so
                // (E, E+1) and (E+2, E+3) sit in registers (q, q+4) and (q+8, q+12)
                // and rotate by the angles of columns E/2 and E/2 + 1
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    f32x4 wt[4];
                    f32x2 cv[4], sv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int e = 64 * (nb >> 1) + 32 * hf + 8 * q + 4 * (nb & 1);
                        wt[q] = *reinterpret_cast<const f32x4*>(nw + e);
                        cv[q] = *reinterpret_cast<const f32x2*>(csr + e / 2);
                        sv[q] = *reinterpret_cast<const f32x2*>(csr + 64 + e / 2);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int gp = 0; gp < 2; ++gp) {
                            const int r0 = q + 8 * gp, r1 = r0 + 4;
                            const float z0 = v[nb][r0] * (inv * wt[q][2 * gp]);
                            const float z1 = v[nb][r1] * (inv * wt[q][2 * gp + 1]);
                            v[nb][r0] = z0 * cv[q][gp] - z1 * sv[q][gp];
                            v[nb][r1] = z1 * cv[q][gp] + z0 * sv[q][gp];
                        }
                }
            } else
            // rotate-half: n-blocks lo = nb and hi = nb + 2 hold dims e and e + 64
#pragma unroll
            for (int lo = 0; lo < 2; ++lo) {
                f32x4 wl[4], wh[4], cv[4], sv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int e = 32 * hf + 8 * q + 4 * lo;
                    wl[q] = *reinterpret_cast<const f32x4*>(nw + e);
                    wh[q] = *reinterpret_cast<const f32x4*>(nw + 64 + e);
                    cv[q] = *reinterpret_cast<const f32x4*>(csr + e);
                    sv[q] = *reinterpret_cast<const f32x4*>(csr + 64 + e);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float zl = v[lo][r] * (inv * wl[r & 3][r >> 2]);
                    const float zh = v[lo + 2][r] * (inv * wh[r & 3][r >> 2]);
                    const float c = cv[r & 3][r >> 2];
                    const float sn = sv[r & 3][r >> 2];
                    v[lo][r] = zl * c - zh * sn;
                    v[lo + 2][r] = zh * c + zl * sn;
                }
            }
        }
        uint16_t* orow = dbase + int64_t(bidx) * a.stride_b + int64_t(row) * a.stride_s;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = 64 * hh + 32 * hf + 8 * q;
                uint4 pk;
                pk.x = uint32_t(bf16_bits(v[2 * hh][q])) | (uint32_t(bf16_bits(v[2 * hh][q + 4])) << 16);
                pk.y = uint32_t(bf16_bits(v[2 * hh][q + 8])) | (uint32_t(bf16_bits(v[2 * hh][q + 12])) << 16);
                pk.z = uint32_t(bf16_bits(v[2 * hh + 1][q])) | (uint32_t(bf16_bits(v[2 * hh + 1][q + 4])) << 16);
                pk.w = uint32_t(bf16_bits(v[2 * hh + 1][q + 8])) | (uint32_t(bf16_bits(v[2 * hh + 1][q + 12])) << 16);
                if (in_range) *reinterpret_cast<uint4*>(orow + e) = pk;
            }
        __builtin_amdgcn_sched_barrier(0);
    }
  };


    // prologue: K-tiles 0 and 1 of the first tile
    load_stage(gw_cur, gx_cur, 0, 0);
    load_stage(gw_cur, gx_cur, 1, 1);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * LOADS) : "memory");
    for (;;) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        // K-tile 1 was requested before this tile began (it overlapped the
        // previous epilogue); K-tile 2 on is requested one region ahead
        region(0, 0, false);
        region(1, 1, true);
        for (int kt = 2; kt < KT; kt += 2) {
            region(kt, 0, true);
            region(kt + 1, 1, true);
        }
        // the next tile's K-tile 0 is in stage 0; request its K-tile 1 into the
        // (free) stage 1 so that it loads during the epilogue
        load_k(KT + 1, 1);
        mfmas(fa_b, fb_b);                          // sub-step 3 of the last K-tile
        // the nops give the last MFMAs' results the wait states an accumulator
        // read needs
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        epilogue(m0, n0);
        if (next >= end) break;
        m0 = m0_next;
        n0 = n0_next;
        gw_cur = gw_nxt;
        gx_cur = gx_nxt;
        next += stride;
        tile_origin(next < end ? next : next - stride, m0_next, n0_next);
        gw_nxt = panel_offset(n0_next);
        gx_nxt = panel_offset(m0_next);
    }
    // drain the requests of the (non-existent) tile after the last one before
    // the workgroup's LDS can be handed to another workgroup
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}

}  // namespace

FusedPlan fused_plan() { return FusedPlan{BM, BN, BK, NT, GROUP_M}; }

// Compute units of the current device (cached per device).
static int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

hipError_t launch_fused(const FusedArgs& a_in, hipStream_t stream) {
    FusedArgs a = a_in;
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    a.group_m = GROUP_M;
    const int tiles = a.tiles_m * a.tiles_n;
    const int grid = tiles < device_cus() ? tiles : device_cus();
    hipLaunchKernelGGL(fused_qkv_kernel, dim3(grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qkvx
