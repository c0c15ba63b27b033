// Fused QKV projection + per-head RMSNorm(Q, K) + RoPE + head-band store, as one
// gfx950 kernel.
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
//    lane l^32, and both RoPE pairings keep their partners in one lane: the
//    whole epilogue is lane-local.
//  * Block tile 256 tokens x 256 columns (two heads), K-step 64, four waves in a
//    2 x 2 grid, each owning one head x 128 tokens: 16 accumulators of 32x32
//    per wave, all 256 AGPRs of the lane.
//  * Operands are K-contiguous and go straight from global memory to LDS
//    (buffer_load ... lds, bounds-checked: rows past M or N read as zero),
//    128 bytes per row per request.  How fast they arrive is set by how many
//    requests a compute unit keeps in flight, and a wait that drains them all
//    once per K-step leaves the memory pipeline idle for a full latency each
//    time.  So the LDS is a ring of five 32 KB buffers, each holding the W or
//    the X half of one K-step: while the MFMAs use K-step k (two buffers), the
//    X half of k+1 and the W half of k+2 load into the buffers K-step k-1 used,
//    and the wait at the end of the step leaves the W half of k+2 in flight.
//    Within a buffer the 16-byte chunks of each 8-row block are XOR-swizzled by
//    the block index, so the fragment reads are free of bank conflicts.
//  * The main loop is a fixed sequence per K-step: 64 MFMA slots in four
//    phases (each phase one 16-deep sub-step of all 16 accumulators), the next
//    sub-step's eight fragment reads right after the first eight MFMAs of a
//    phase, and the 16 load instructions in the other half of the slots (a
//    load holds the wave's issue for ~24 cycles).  MFMAs and
//    fragment reads are written as inline assembly with explicit
//    lgkmcnt waits: the buffer a read uses is only known at run time, and
//    the compiler, unable to tell it from the buffers being loaded, would
//    otherwise wait for every load in flight before each read.
//  * Persistent: one workgroup per CU, and the K-steps of a workgroup's
//    consecutive output tiles form one continuous load stream, so the next
//    tile's first K-steps are in flight while the current tile's epilogue
//    runs.  The 8 XCDs (workgroup b runs on XCD b % 8) take consecutive ranges
//    of a tile order that walks groups of tile rows column by column, so the
//    tiles an XCD runs together share X and W panels in its L2.  Each XCD runs
//    at its own clock under this load, so past two fixed rounds workgroups
//    claim tiles one at a time from per-XCD counters (then from the other
//    XCDs' ranges), and all XCDs finish together.
//  * Epilogue: Q/K norm and RoPE in registers, with the weights and cos/sin
//    values loaded one q ahead; stores are transposed within groups of four
//    lanes so that each store instruction writes whole 64-byte runs, and go
//    out once per m-block.
#include "qkvx_internal.h"

namespace qkvx {
namespace {

constexpr int BM = 256;        // tokens per tile
constexpr int BN = 256;        // output columns per tile (two heads)
constexpr int BK = 64;         // K per step (128 bytes of each operand row)
constexpr int NT = 256;        // threads: four waves
constexpr int GROUP_M = 8;     // tile rows walked together in the tile order
constexpr int NXCD = 8;
constexpr int NBUF = 5;        // ring of half-step buffers
constexpr int BUF_CHUNKS = 2048;    // 16-byte chunks per buffer: 256 rows x 128 bytes
constexpr int HLOADS = 8;      // load instructions per wave per half step

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte chunk index, within one buffer, of chunk c (0..7) of tile row r:
// block r / 8 holds rows 8 (r / 8) .. + 7, 128 bytes each, with chunk c of a
// row at position c ^ (block % 8).  Fragment reads of one chunk by lanes whose
// rows lie in eight consecutive blocks therefore hit eight different 16-byte
// bank groups.
__device__ __forceinline__ int lds_pos(int r, int c) {
    const int b = r >> 3;
    return b * 64 + (r & 7) * 8 + (c ^ (b & 7));
}

// Row of a wave's 128-row range that MFMA row i (0..31) of 32-row block blk
// maps to.  Lanes i..i+7 read rows 8 apart, i.e. in eight consecutive blocks.
__device__ __forceinline__ int mfma_row(int blk, int i) {
    return 64 * (blk >> 1) + 8 * (i & 7) + 4 * (blk & 1) + (i >> 3);
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

// Two floats rounded to bf16 (nearest even) and packed, lo in bits 0-15: one
// v_cvt_pk_bf16_f32.  (Converting each float alone and packing the halves
// costs three instructions per pair.)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Accumulators are read with explicit v_accvgpr_read so that the compiler
// never copies all 256 of them into VGPRs at once (there is no room).
__device__ __forceinline__ float acc_read(const float& a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// Lane exchange within groups of four lanes (DPP quad permutation).
template <int CTRL>
__device__ __forceinline__ uint32_t quad_perm(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap2 = 2 | 3 << 2 | 0 << 4 | 1 << 6;   // lane k reads lane k ^ 2
constexpr int kQuadSwap1 = 1 | 0 << 2 | 3 << 4 | 2 << 6;   // lane k reads lane k ^ 1
template <int I>
constexpr int quad_bcast() { return I | I << 2 | I << 4 | I << 6; }   // every lane reads lane I

// Transpose of 4 x 4 elements of 16 bytes within each group of four lanes:
// on entry lane k holds pieces r[0..3] of its own row, on return r[i] holds
// piece k of the row of lane i of the group.  Two exchange stages, between
// lanes k and k ^ 2 (pieces with bit 1 set) and between k and k ^ 1 (bit 0).
__device__ __forceinline__ void quad_transpose(uint4 (&r)[4], int k) {
    const bool b1 = (k >> 1) & 1, b0 = k & 1;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        uint32_t* lo = reinterpret_cast<uint32_t*>(&r[jj]);
        uint32_t* hi = reinterpret_cast<uint32_t*>(&r[jj + 2]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t recv = quad_perm<kQuadSwap2>(b1 ? lo[c] : hi[c]);
            if (b1) lo[c] = recv; else hi[c] = recv;
        }
    }
#pragma unroll
    for (int jj = 0; jj < 4; jj += 2) {
        uint32_t* lo = reinterpret_cast<uint32_t*>(&r[jj]);
        uint32_t* hi = reinterpret_cast<uint32_t*>(&r[jj + 1]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t recv = quad_perm<kQuadSwap1>(b0 ? lo[c] : hi[c]);
            if (b0) lo[c] = recv; else hi[c] = recv;
        }
    }
}

template <int N>
__device__ __forceinline__ void wait_lgkm() {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// ROWS_CHECKED: M < BM, so the single tile row reads X rows past M, which must
// come from the buffer's range check (zeros).  Otherwise the last tile row and
// the last tile column are moved back to end at M and N, so that every operand
// row a tile reads exists; the rows (heads) it shares with the previous tile
// are computed again with the same instruction sequence and stored again with
// the same bits.
template <bool ROWS_CHECKED, bool ROPE_IL>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void fused_qkv_kernel(FusedArgs a) {
    // K-step g of the stream occupies W half 2g and X half 2g + 1; half h
    // lives in buffer h % 5.
    __shared__ uint4 ring[NBUF * BUF_CHUNKS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wn = wave & 1;      // which head of the tile
    const int wm = wave >> 1;     // which 128 tokens of the tile

    // ---- tile schedule ---------------------------------------------------------
    // The logical tile order is split into queues, one per XCD (workgroups b
    // with b % 8 == x run on XCD x), or a single queue for a grid that is not
    // a multiple of 8.  Queue x holds a contiguous share of the order; with
    // readiness words the order is destination-major and is shared out one
    // destination at a time (queue x: its share of destination 0's tiles,
    // then of destination 1's, ...), so that destinations complete one after
    // another while each XCD keeps runs of neighbouring tiles.  A queue's
    // workgroups take its first two rounds (one tile each per round) in a
    // fixed order; with tile-claim counters the rest is claimed one tile at a
    // time (the workgroup's own queue first, then the others once it is used
    // up), so that XCDs running at a higher clock take more tiles and all
    // finish together.  Without counters the workgroups walk their queue a
    // round at a time.
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int total = a.tiles_m * a.tiles_n;
    const bool by_xcd = G % NXCD == 0;
    const int nq = by_xcd ? NXCD : 1;
    const bool claim = a.sched != nullptr;
    // span: the tiles shared out among the queues at a time (one destination's
    // tiles, world of them in all, or the whole order)
    const int span = a.ready && a.dest_cols > 0 ? a.tiles_m * 3 * a.dest_cols : total;
    const int nspan = total / span;
    const int per = span / nq, rem = span % nq;
    auto share_start = [&](int x) { return x * per + min(x, rem); };
    auto share_len = [&](int x) { return per + (x < rem ? 1 : 0); };
    auto qlen = [&](int x) { return nspan * share_len(x); };
    // logical tile at position i < qlen(x) of queue x
    auto qtile = [&](int x, int i) {
        const int len = share_len(x);
        const int sp = i / len;
        return sp * span + share_start(x) + (i - sp * len);
    };
    const int xcd = by_xcd ? bid % NXCD : 0;        // the workgroup's queue
    const int stride = by_xcd ? G / NXCD : G;       // workgroups per queue
    const int qfirst = by_xcd ? bid / NXCD : bid;   // its first position in the queue
    // Once a workgroup has claimed its last tile it counts itself finished;
    // the last one to do so zeroes the counters for the next launch (every
    // claim of this launch has returned by then).
    auto finish = [&]() {
        if (claim && threadIdx.x == 0) {
            const unsigned int old = __hip_atomic_fetch_add(a.sched + NXCD, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
            if (old == unsigned(G - 1)) {
                for (int v = 0; v <= NXCD; ++v)
                    __hip_atomic_store(a.sched + v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };
    if (qfirst >= qlen(xcd)) {
        finish();
        return;
    }
    const int first = qtile(xcd, qfirst);
    const int K = a.K;
    // With readiness words the order is destination-major: the tiles holding
    // destination d's heads (dest_cols columns in each of q, k, v) come before
    // those of d + 1, so early destinations are complete early.
    // n_own: the first output column the tile is responsible for (before the
    // move back), which decides the heads it counts in the readiness words.
    auto tile_origin = [&](int l, int& m0, int& n0, int& n_own) {
        int tm, tn;
        if (a.ready && a.dest_cols > 0) {
            const int per_dest = a.tiles_m * 3 * a.dest_cols;
            const int d = l / per_dest;
            int c;
            tile_coords(l - d * per_dest, a.tiles_m, 3 * a.dest_cols, a.group_m, tm, c);
            const int p = c / a.dest_cols;
            tn = p * a.part_cols + d * a.dest_cols + (c - p * a.dest_cols);
        } else {
            tile_coords(l, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
        }
        m0 = tm * BM;
        n0 = tn * BN;
        n_own = n0;
        if (!ROWS_CHECKED && m0 + BM > a.M) m0 = a.M - BM;
        if (n0 + BN > a.N) n0 = a.N - BN;
    };

    // ---- global -> LDS: direct loads (buffer_load ... lds) ----------------------
    // Instruction i of wave w fills block b = 4 i + w of a half: lane L brings
    // the chunk stored at position L % 8 of row L / 8 of the block, i.e. chunk
    // (L % 8) ^ (b % 8) of panel row 8 b + L / 8; the eight lanes of a row fetch
    // its whole 128-byte segment.  b % 8 = 4 (i % 2) + w, so even and odd
    // instructions use two lane offsets that differ in bit 6.
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.w, (short)0, int(uint32_t(a.N) * uint32_t(K) * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, (short)0, int(uint32_t(a.M) * uint32_t(K) * 2u), 0x00020000);
    // byte sizes are below 2^32 (checked on the host); reads past them return 0
    const uint32_t rowbytes = uint32_t(K) * 2u;
    const int wv = wave;
    const uint32_t lrow = uint32_t(8 * wv + (lane >> 3));
    const uint32_t lchunk = uint32_t((lane & 7) ^ wv) * 16u;
    // this lane's byte offset of K-step 0 of a panel at row origin (even
    // instructions; odd ones: ^ 64)
    auto panel_offset = [&](int origin) {
        return (uint32_t(origin) + lrow) * rowbytes + lchunk;
    };

    // ---- fragment reads: lane i%32 owns MFMA row i%32 of each 32-row block ----
    // Sub-step ks reads chunk 2 ks + hf of each row: the position of chunk hf
    // with bits 1-2 flipped by 2 ks.  Byte offsets within a buffer:
    const int fr = lane & 31;
    const int hf = lane >> 5;
    uint32_t wo[4][4], xo[4][4];                           // [ks][block]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            wo[ks][b] = uint32_t(lds_pos(wn * 128 + mfma_row(b, fr), hf) ^ (2 * ks)) * 16u;
            xo[ks][b] = uint32_t(lds_pos(wm * 128 + mfma_row(b, fr), hf) ^ (2 * ks)) * 16u;
        }
    typedef __attribute__((address_space(3))) uint4 lds_uint4;
    lds_uint4* ring3 = (lds_uint4*)ring;
    const uint32_t ring0 = uint32_t(reinterpret_cast<uintptr_t>(ring3));

    f32x16 acc[4][4];
    // fragments of one sub-step: four 32-row blocks of W (A operand) and of X
    // (B operand); two sets, A and B
    bf16x8 fa_a[4], fb_a[4], fa_b[4], fb_b[4];

    // One MFMA on accumulator (nb, mb); `init`: the tile's first product, with
    // a zero accumulator input (no separate zeroing).
    auto mfma1 = [&](int nb, int mb, const bf16x8& fa, const bf16x8& fb, bool init) {
        if (init)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                         : "=a"(acc[nb][mb]) : "v"(fa), "v"(fb));
        else
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+a"(acc[nb][mb]) : "v"(fa), "v"(fb));
    };
    // A fragment read.  Its result may only be used after a wait_lgkm that
    // covers it: the compiler does not track it, and every use below is an
    // MFMA placed after such a wait.
    auto lds_read = [&](bf16x8& dst, uint32_t addr) {
        asm volatile("ds_read_b128 %0, %1" : "=v"(dst) : "v"(addr));
    };

    const int KT = K / BK;
    // Panels of the current tile and of this workgroup's next tile; past its
    // last tile the "next" requests re-read the current tile (in bounds, unused).
    // nxt: the tile after the current one, or -1.
    int m0, n0, m0_next, n0_next, own, own_next;
    tile_origin(first, m0, n0, own);
    int qnxt = qfirst + stride;                      // queue position of nxt (fixed order)
    int nxt = qnxt < qlen(xcd) ? qtile(xcd, qnxt) : -1;
    tile_origin(nxt >= 0 ? nxt : first, m0_next, n0_next, own_next);
    uint32_t gw_cur = panel_offset(n0), gx_cur = panel_offset(m0);
    uint32_t gw_nxt = panel_offset(n0_next), gx_nxt = panel_offset(m0_next);

    // Load instruction i (0..7) of the W or X half of K-step kidx of the
    // stream (kidx >= KT: the next output tile) into buffer buf.
    auto load_one = [&](bool is_w, int i, int kidx, int buf) {
        const bool nx = kidx >= KT;
        const uint32_t g0 = is_w ? (nx ? gw_nxt : gw_cur) : (nx ? gx_nxt : gx_cur);
        const uint32_t kb = uint32_t(nx ? kidx - KT : kidx) * BK * 2u;
        const uint32_t flip = (i & 1) ? 64u : 0u;
        const uint32_t roff = uint32_t(32 * i) * rowbytes;
        lds_uint4* dst = ring3 + buf * BUF_CHUNKS + (4 * i + wv) * 64;
        // The buffer's range check covers the VGPR offset but not the SGPR
        // offset.  When rows past M are read (ROWS_CHECKED) the row goes into
        // the VGPR offset so that they read as zeros; otherwise every row read
        // exists and the instruction's row step rides in the SGPR offset with
        // the K offset, which keeps the loop free of address arithmetic.
        const uint32_t voff = ROWS_CHECKED ? (g0 ^ flip) + roff : (g0 ^ flip);
        const uint32_t soff = ROWS_CHECKED ? kb : roff + kb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_w ? rw : rx,
                                                 (__attribute__((address_space(3))) void*)dst, 16,
                                                 voff, soff, 0, 0);
    };

    // ---- main loop ------------------------------------------------------------
    // K-step kt of the current tile, W half in buffer pw.  64 MFMA slots in
    // four phases of 16 (phase 0: set B, the previous K-step's sub-step 3; 1:
    // set A, sub-step 0; 2: set B, sub-step 1; 3: set A, sub-step 2).  After
    // slot j < 8 of phase p comes fragment read j of sub-step p into the other
    // set (that set's MFMAs all issued in the previous phase); after slots
    // j = 8, 10, 12, 14 one of the 16 load instructions of the X half of
    // K-step kt+1 and the W half of K-step kt+2, into the two buffers K-step
    // kt-1 used.
    // The step ends waiting for all but the last eight loads (the W half of
    // kt+2, which stays in flight) and for the reads, then the barrier.  A
    // tile's first step has no phase 0: its sub-step-0 fragments are read
    // up front and phase 1 starts the accumulators.
    int pw = 0;
    auto step = [&](int kt, bool first_of_tile) {
        const int px = pw == 4 ? 0 : pw + 1;
        const int bx1 = pw >= 2 ? pw - 2 : pw + 3;       // (pw + 3) % 5
        const int bw2 = pw >= 1 ? pw - 1 : 4;            // (pw + 4) % 5
        const uint32_t wb = ring0 + uint32_t(pw) * (BUF_CHUNKS * 16);
        const uint32_t xb = ring0 + uint32_t(px) * (BUF_CHUNKS * 16);
        const int i0 = first_of_tile ? 16 : 0;
        if (first_of_tile) {
#pragma unroll
            for (int b = 0; b < 4; ++b) lds_read(fa_a[b], wb + wo[0][b]);
#pragma unroll
            for (int b = 0; b < 4; ++b) lds_read(fb_a[b], xb + xo[0][b]);
        }
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            if (i < i0) continue;
            const int ph = i >> 4, j = i & 15;
            const int nb = j >> 2, mb = j & 3;
            // The first row (nb 0) of a phase needs read 4 + mb of the previous
            // phase's eight, in order; the j reads issued in this phase so far
            // come after them: at most 3 - mb + j = 3 may be outstanding.
            if (ph > 0 && j < 4) wait_lgkm<3>();
            if (ph & 1)
                mfma1(nb, mb, fa_a[nb], fb_a[mb], first_of_tile && ph == 1);
            else
                mfma1(nb, mb, fa_b[nb], fb_b[mb], false);
            // Loads go only into slots without a fragment read (j >= 8): a
            // load instruction holds the wave's issue for ~24 cycles while it
            // sends 64 addresses, which must fit beside the slot's MFMA.
            // Steady steps use j = 8, 10, 12, 14 of every phase; a tile's
            // first step every slot j >= 8 of phases 1 and 2.
            const int v = first_of_tile ? ((ph - 1) * 8 + (j - 8)) : (ph * 4 + (j - 8) / 2);
            if (j >= 8 && (first_of_tile ? ph <= 2 : (j & 1) == 0) && v < 2 * HLOADS) {
                if (v < HLOADS) load_one(false, v, kt + 1, bx1);
                else load_one(true, v - HLOADS, kt + 2, bw2);
            }
            if (j < 8) {
                bf16x8* fa = (ph & 1) ? fa_b : fa_a;
                bf16x8* fb = (ph & 1) ? fb_b : fb_a;
                if (j < 4) lds_read(fa[j], wb + wo[ph][j]);
                else lds_read(fb[j - 4], xb + xo[ph][j - 4]);
            }
        }
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(HLOADS) : "memory");
        pw = pw >= 3 ? pw - 3 : pw + 2;                  // (pw + 2) % 5
    };

    // ---- epilogue: one head (128 columns) per wave ----------------------------
    // Accumulator register reg of n-block nb in lane-half hf holds head dim
    //   e = 64 (nb / 2) + 32 hf + 8 (reg % 4) + 4 (nb % 2) + reg / 4
    // of the token of MFMA column fr of m-block mb, tile token
    //   wm * 128 + mfma_row(mb, fr).
    // Registers q, q+4, q+8, q+12 hold four consecutive dims; n-blocks 2h and
    // 2h+1 continue each other (16 bytes of bf16); n-block nb+2 holds e + 64.
    // Each m-block is read twice (sum of squares, then the outputs, four dims
    // per n-block at a time), which keeps the VGPRs in use small.
    //
    // Memory: the norm weights and cos/sin values of (m-block, q) are loaded
    // while the previous q is computed; an m-block's stores go out after the
    // next block's first loads.  Vector memory operations retire in order, so
    // a wait for loads also waits for every older store: stores are therefore
    // grouped (one group per m-block) and made of whole 64-byte runs.
    // Per (m-block, q) a Q/K wave needs 4 weight vectors and 2 + 2 cos/sin
    // vectors; they are loaded one q ahead into the other of two buffers.
    //   Wq[i] = w[64 (i / 2) + 32 hf + 8 q + 4 (i % 2)]          (i < 4)
    //   rotate-half: Cq[lo] = cs[row][32 hf + 8 q + 4 lo], Sq at + 64
    //   interleaved: Cq[hi] = cs[row][32 hi + 16 hf + 4 q],  Sq at + 64
    f32x4 Wb[2][4], Cb[2][2], Sb[2][2];
    auto load_tables = [&](const float* nw, int row, int q, int buf) {
        const float* csr = a.cs + int64_t(row) * 128;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Wb[buf][i] = *reinterpret_cast<const f32x4*>(nw + 64 * (i >> 1) + 32 * hf + 8 * q +
                                                         4 * (i & 1));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int off = ROPE_IL ? 32 * i + 16 * hf + 4 * q : 32 * hf + 8 * q + 4 * i;
            Cb[buf][i] = *reinterpret_cast<const f32x4*>(csr + off);
            Sb[buf][i] = *reinterpret_cast<const f32x4*>(csr + 64 + off);
        }
    };
    // The first (m-block 0, q 0) values of a Q/K wave's tile, issued before
    // the tile's last K-step: that step's end-of-step wait then covers them,
    // instead of the epilogue waiting for them behind the ring loads of the
    // next tile (vector memory operations retire in order).
    auto first_tables = [&](int m0, int n0) {
        const int ncol = n0 + wn * 128;
        if (ncol >= a.N) return;
        const int p = ncol / a.hidden;
        if (p == 2) return;
        const int m_tile = m0 + wm * 128 + mfma_row(0, fr);
        const int m = m_tile < a.M ? m_tile : a.M - 1;
        const int s = m - (m / a.s_local) * a.s_local;
        load_tables(p == 0 ? a.wq : a.wk, a.row0 + s, 0, 0);
    };

    auto epilogue = [&](int m0, int n0) {
    const int ncol = n0 + wn * 128;
    if (ncol >= a.N) return;
    const int p = ncol / a.hidden;                 // 0 q, 1 k, 2 v
    const int h = (ncol - p * a.hidden) >> 7;
    const int d = h / a.local_heads;
    const int j = h - d * a.local_heads;
    uint16_t* dbase = a.slot + int64_t(d) * a.region_elems + int64_t(p) * a.part_stride +
                      int64_t(j) * a.stride_h;
    // token of m-block mb: tokens past M (ragged last tile) are computed on
    // token M - 1 and not stored
    auto token_row = [&](int mb, bool& in_range) {
        const int m_tile = m0 + wm * 128 + mfma_row(mb, fr);
        in_range = m_tile < a.M;
        const int m = in_range ? m_tile : a.M - 1;
        const int bidx = m / a.s_local;
        const int s = m - bidx * a.s_local;
        return make_int2(bidx, a.row0 + s);   // batch, sequence row == position
    };
    // Stores of one m-block.  Lane (fr, hf) holds 16-byte pieces q = 0..3 of
    // dims 64 hh + 32 hf + 8 q of its token; after a transpose within each
    // group of four lanes (four tokens), store i of a group writes the four
    // pieces of one token's 64 contiguous bytes, so that each store makes 16
    // requests of 64 bytes instead of 64 of 16.
    auto store_block = [&](uint16_t* orow, bool in_range, const uint4* out) {
        const int k = fr & 3;
        uint4 r[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int q = 0; q < 4; ++q) r[hh][q] = out[2 * q + hh];
            quad_transpose(r[hh], k);
        }
        // store i: the row of group lane i (its pointer and range flag read
        // from that lane), this lane's piece k
        const uint64_t rowp = reinterpret_cast<uint64_t>(orow);
        const uint32_t rlo = uint32_t(rowp), rhi = uint32_t(rowp >> 32), ok = in_range;
        const uint64_t off = uint64_t(64 * hf + 16 * k);          // bytes
        auto put = [&](uint32_t lo, uint32_t hi, uint32_t f, int i) {
            if (f) {
                uint16_t* dst = reinterpret_cast<uint16_t*>(((uint64_t(hi) << 32) | lo) + off);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    *reinterpret_cast<uint4*>(dst + 64 * hh) = r[hh][i];
            }
        };
        put(quad_perm<quad_bcast<0>()>(rlo), quad_perm<quad_bcast<0>()>(rhi),
            quad_perm<quad_bcast<0>()>(ok), 0);
        put(quad_perm<quad_bcast<1>()>(rlo), quad_perm<quad_bcast<1>()>(rhi),
            quad_perm<quad_bcast<1>()>(ok), 1);
        put(quad_perm<quad_bcast<2>()>(rlo), quad_perm<quad_bcast<2>()>(rhi),
            quad_perm<quad_bcast<2>()>(ok), 2);
        put(quad_perm<quad_bcast<3>()>(rlo), quad_perm<quad_bcast<3>()>(rhi),
            quad_perm<quad_bcast<3>()>(ok), 3);
    };
    auto pack = [&](const float (&v)[4][4], uint4* out2) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            uint4 pk;
            pk.x = bf16_pair(v[2 * hh][0], v[2 * hh][1]);
            pk.y = bf16_pair(v[2 * hh][2], v[2 * hh][3]);
            pk.z = bf16_pair(v[2 * hh + 1][0], v[2 * hh + 1][1]);
            pk.w = bf16_pair(v[2 * hh + 1][2], v[2 * hh + 1][3]);
            out2[hh] = pk;
        }
    };

    if (p == 2) {
        // V: rounding and placement only
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            bool in_range;
            const auto br = token_row(mb, in_range);
            uint16_t* orow = dbase + int64_t(br.x) * a.stride_b + int64_t(br.y) * a.stride_s;
            uint4 out[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4][4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) v[nb][g] = acc_read(acc[nb][mb][q + 4 * g]);
                pack(v, out + 2 * q);
            }
            store_block(orow, in_range, out);
        }
        __builtin_amdgcn_sched_barrier(0);
        return;
    }

    // m-block 0, q 0 of the tables are already loaded (first_tables)
    const float* nw = p == 0 ? a.wq : a.wk;
    int rows[4];
    bool in_range[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const auto br = token_row(mb, in_range[mb]);
        rows[mb] = br.y;
    }
    auto load_q = [&](int mb, int q, int buf) { load_tables(nw, rows[mb], q, buf); };

#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        // RMSNorm over the head's 128 values: 64 here, 64 in lane ^ 32
        float ss = 0.f;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float t = acc_read(acc[nb][mb][r]);
                ss += t * t;
            }
        ss += __shfl_xor(ss, 32);
        const float inv = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
        uint4 out[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int cur = (4 * mb + q) & 1;
            if (4 * mb + q < 15) load_q(q < 3 ? mb : mb + 1, (q + 1) & 3, cur ^ 1);
            // v[nb][g] = dim e(nb, q) + g, g = 0..3 (registers q + 4 g)
            float v[4][4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) v[nb][g] = acc_read(acc[nb][mb][q + 4 * g]);
            if (ROPE_IL) {
                // pairs (2i, 2i+1) = dims (E, E+1) and (E+2, E+3) of each
                // n-block, E = e(nb, q), rotated by the angles of table columns
                // E/2 and E/2 + 1
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const f32x4 wt = Wb[cur][nb];
                    const f32x4 cv = Cb[cur][nb >> 1], sv = Sb[cur][nb >> 1];
#pragma unroll
                    for (int gp = 0; gp < 2; ++gp) {
                        const float z0 = v[nb][2 * gp] * (inv * wt[2 * gp]);
                        const float z1 = v[nb][2 * gp + 1] * (inv * wt[2 * gp + 1]);
                        const float c = cv[2 * (nb & 1) + gp], sn = sv[2 * (nb & 1) + gp];
                        v[nb][2 * gp] = z0 * c - z1 * sn;
                        v[nb][2 * gp + 1] = z1 * c + z0 * sn;
                    }
                }
            } else {
                // rotate-half: n-blocks lo and lo + 2 hold dims e and e + 64
#pragma unroll
                for (int lo = 0; lo < 2; ++lo) {
                    const f32x4 wl = Wb[cur][lo], wh = Wb[cur][2 + lo];
                    const f32x4 cv = Cb[cur][lo], sv = Sb[cur][lo];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float zl = v[lo][g] * (inv * wl[g]);
                        const float zh = v[lo + 2][g] * (inv * wh[g]);
                        v[lo][g] = zl * cv[g] - zh * sv[g];
                        v[lo + 2][g] = zh * cv[g] + zl * sv[g];
                    }
                }
            }
            pack(v, out + 2 * q);
            __builtin_amdgcn_sched_barrier(0);
        }
        // this block's stores go out after the next block's first loads
        const auto br = token_row(mb, in_range[mb]);
        uint16_t* orow = dbase + int64_t(br.x) * a.stride_b + int64_t(br.y) * a.stride_s;
        store_block(orow, in_range[mb], out);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

    // claim state (thread 0 only): the queue counter being drawn from, and how
    // many counters were found used up
    int cvict = xcd, ctried = 0;

    // prologue: W and X halves of K-step 0 and the W half of K-step 1
#pragma unroll
    for (int i = 0; i < HLOADS; ++i) load_one(true, i, 0, 0);
#pragma unroll
    for (int i = 0; i < HLOADS; ++i) load_one(false, i, 0, 1);
#pragma unroll
    for (int i = 0; i < HLOADS; ++i) load_one(true, i, 1, 2);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(HLOADS) : "memory");
    for (;;) {
        step(0, true);
        for (int kt = 1; kt < KT - 1; ++kt) step(kt, false);
        first_tables(m0, n0);
        step(KT - 1, false);
        // sub-step 3 of the last K-step (its fragments arrived before the barrier)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) mfma1(nb, mb, fa_b[nb], fb_b[mb], false);
        // the nops give the last MFMAs' results the wait states an accumulator
        // read needs
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        // Claim the tile after nxt: the counter's reply is only needed after
        // the epilogue, whose own memory waits cover it.
        const bool claiming = claim && nxt >= 0;
        unsigned int reply = 0;
        if (claiming && threadIdx.x == 0)
            reply = __hip_atomic_fetch_add(a.sched + cvict, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        epilogue(m0, n0);
        if (a.ready) {
            // publish: once all four waves' stores of this tile are complete,
            // release them at agent scope and count the tile's two heads (two
            // waves each) for their destinations
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            if (wave == 0) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                if (lane < 2) {
                    const int ncol = n0 + lane * 128;
                    if (ncol < a.N && ncol >= own) {
                        const int p = ncol / a.hidden;
                        const int h = (ncol - p * a.hidden) >> 7;
                        __hip_atomic_fetch_add(a.ready + h / a.local_heads, 2ull,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
        }
        if (nxt < 0) break;
        int after;
        if (claiming) {
            // Thread 0 turns the reply into a tile (claiming from the next
            // XCDs' counters while the current one's range is used up) and
            // hands it to the other waves through the first word of the buffer
            // the last K-step's W half used: it is free until the next tile's
            // first step loads into it, after the second barrier.
            const uint32_t mail = ring0 + uint32_t(pw >= 2 ? pw - 2 : pw + 3) * (BUF_CHUNKS * 16);
            if (threadIdx.x == 0) {
                int t = -1;
                for (;;) {
                    const int idx = 2 * stride + int(reply);
                    if (idx < qlen(cvict)) {
                        t = qtile(cvict, idx);
                        break;
                    }
                    if (++ctried == nq) break;
                    cvict = cvict == nq - 1 ? 0 : cvict + 1;
                    reply = __hip_atomic_fetch_add(a.sched + cvict, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                }
                asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(mail), "v"(t)
                             : "memory");
            }
            int got;
            asm volatile("s_barrier\n\tds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                         : "=v"(got) : "v"(mail) : "memory");
            after = __builtin_amdgcn_readfirstlane(got);
        } else {
            qnxt += stride;
            after = qnxt < qlen(xcd) ? qtile(xcd, qnxt) : -1;
        }
        m0 = m0_next;
        n0 = n0_next;
        own = own_next;
        gw_cur = gw_nxt;
        gx_cur = gx_nxt;
        // past the last tile the "next" requests re-read the current one
        tile_origin(after >= 0 ? after : nxt, m0_next, n0_next, own_next);
        nxt = after;
        gw_nxt = panel_offset(n0_next);
        gx_nxt = panel_offset(m0_next);
    }
    finish();
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
    // with readiness words one CU per XCD stays free, so that wait kernels on
    // other streams always find room while this grid runs
    const int all_cus = device_cus();
    const int cus = a.ready && all_cus > 2 * NXCD ? all_cus - NXCD : all_cus;
    const int grid = tiles < cus ? tiles : cus;
    auto kernel = a.M < BM ? (a.rope_interleaved ? fused_qkv_kernel<true, true>
                                                 : fused_qkv_kernel<true, false>)
                           : (a.rope_interleaved ? fused_qkv_kernel<false, true>
                                                 : fused_qkv_kernel<false, false>);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qkvx
