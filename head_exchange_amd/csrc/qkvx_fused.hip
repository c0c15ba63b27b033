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
//    v_mfma_f32_16x16x32_bf16.  Under the chip's power limit the kernel runs
//    at a 13 % higher clock with this form than with v_mfma_f32_32x32x16_bf16
//    (it moves half the accumulator bytes per multiply-add), which more than
//    pays for the load issue the longer form would hide.  In the 16x16
//    accumulator layout a lane owns one column (here: one token) and four
//    rows (here: head dims) of a block, and the four lanes l + 16 g share the
//    token.  A wave's 128-row
//    n-range is exactly one head, so the RMS reduction over the head is a
//    register sum plus two exchanges, and both RoPE pairings keep their
//    partners in one lane; with the operand rows staged in a fixed
//    permutation, each lane holds four 16-byte runs of its token's head
//    vector and the four lanes of a token together 64-byte runs.
//  * Block tile 256 tokens x 256 columns (two heads), K-step 64, four waves in a
//    2 x 2 grid, each owning one head x 128 tokens: 64 accumulators of 16x16
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
//    Within a buffer the 16-byte chunks of each row are XOR-swizzled by a
//    function of the row, so the fragment reads are free of bank conflicts.
//  * The main loop is a fixed sequence per K-step: 128 MFMA slots that give
//    each of the 64 accumulators its two 32-deep multiply-adds back to back
//    (the chip holds a higher clock when an accumulator is written and read
//    again at once: 6-7 % faster per kernel than one multiply-add per
//    accumulator in turn), with the whole K-step's fragments in registers
//    while the next K-step's fragment reads are spread over the slots (a W
//    block right after its last MFMA), and 16 load instructions in slots
//    without a read (a load holds the wave's issue for ~24 cycles).  MFMAs
//    and fragment reads are written as inline assembly with explicit lgkmcnt
//    waits: the buffer a read uses is only known at run time, and the
//    compiler, unable to tell it from the buffers being loaded, would
//    otherwise wait for every load in flight before each read.
//  * Persistent: one workgroup per CU, and the K-steps of a workgroup's
//    consecutive output tiles form one continuous load stream, so the next
//    tile's first K-step is already in LDS when the current tile's epilogue
//    runs.  The 8 XCDs (workgroup b runs on XCD b % 8) each own a run of tile
//    rows and walk it column by column, all starting at column 0 (row bands
//    when X is larger than the MALL; in a band of few rows two or four XCDs
//    share a run, each walking its own range of columns from that range's
//    first): the tiles an XCD runs together share X and W panels in its L2,
//    and the XCDs stream the W column panels in step, so that each comes
//    from HBM about once and is then read from the MALL.
//    Each XCD runs at its own clock under this load, so past two fixed rounds
//    workgroups claim tiles one at a time from per-XCD counters (then from
//    the other XCDs' queues, the fullest first), and all XCDs finish together.
//  * Epilogue: Q/K norm and RoPE in registers, with the weights and cos/sin
//    values loaded one step ahead (the first at the epilogue's start);
//    lanes of tokens 16 apart trade pieces so that each (nontemporal) store
//    instruction writes whole 128-byte lines, and an m-block's stores go out
//    together.
#include <mutex>
#include <type_traits>

#include "qkvx_internal.h"

namespace qkvx {

// Device scratch of qkvx_forward_noalloc: the tile-claim counters of its
// launches, in memory the library never allocates.  Every GPU holds its own
// copy, shared by all such calls on that GPU, for the life of the process.
// Host code must not take this name for a device address: it uses the
// per-device address from scratch_address().
static __device__ __align__(256) unsigned int scratch[kScratchWords];

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
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS layout of one buffer: 256 rows of 128 bytes (eight 16-byte chunks); row
// r sits at 16-byte position 8 r, with chunk c of the row at slot c ^ swz(r),
//   swz(r) = 2 ((r / 8) % 4) + (r / 2) % 2.
// The 16 lanes that read one chunk of a fragment at a time take rows
// mfma_row(blk, 0..15): four 8-row blocks (r / 8 % 4 = 0..3) x rows 4 t + 0..3
// of each, i.e. both row parities and both values of (r / 2) % 2, so the
// (row parity, swizzled slot) pairs, which select the 16-byte bank group of a
// read, are all different: the fragment reads are free of bank conflicts.
__device__ __forceinline__ int lds_swz(int r) { return 2 * ((r >> 3) & 3) + ((r >> 1) & 1); }

// Row of a wave's 128-row range that row i (0..15) of 16-row MFMA block blk
// (0..7) maps to: 32 (blk / 2) + 8 (i / 4) + 4 (blk % 2) + i % 4.  Accumulator
// register r of lane group g (lanes 16 g .. 16 g + 15) holds block row
// i = 4 g + r, so blocks 2h and 2h + 1 give lane group g the eight consecutive
// rows 32 h + 8 g .. + 7, and block blk + 4 holds the rows 64 further on.
__device__ __forceinline__ int mfma_row(int blk, int i) {
    return 32 * (blk >> 1) + 8 * (i >> 2) + 4 * (blk & 1) + (i & 3);
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

// Sum of v over the four lanes l ^ 16 k (k = 0..3) that share l % 16: two
// permlane swaps (lanes 16-31 <-> 0-15 and 48-63 <-> 32-47; then the two
// 32-lane halves), each followed by an add of the pair, which is the same sum
// in the same order as two xor-shuffle steps, without an LDS round trip.
__device__ __forceinline__ float sum_lane_groups(float v) {
    const unsigned int u = __float_as_uint(v);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float s = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const unsigned int w = __float_as_uint(s);
    const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// A 16-byte output piece, stored nontemporally: the receive slots stand in
// for other ranks' memory and are not read again by this kernel (on the same
// box this measured 0.5-2 % faster than plain stores).
__device__ __forceinline__ void store_stream(uint16_t* p, const uint4& v) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

// The value of lane fi ^ 8 of this lane's 16-lane row (DPP row rotate by 8).
__device__ __forceinline__ unsigned int swap8(unsigned int v) {
    return unsigned(__builtin_amdgcn_update_dpp(0, int(v), 0x128, 0xf, 0xf, false));
}

// One DPP move with a bank mask: lanes 8-15 of each 16-lane row (banks 2, 3)
// take v from lane fi ^ 8 and lanes 0-7 keep `keep` (take_hi); take_lo the
// other way round.
__device__ __forceinline__ unsigned int take_hi(unsigned int keep, unsigned int v) {
    return unsigned(__builtin_amdgcn_update_dpp(int(keep), int(v), 0x128, 0xf, 0xc, false));
}
__device__ __forceinline__ unsigned int take_lo(unsigned int keep, unsigned int v) {
    return unsigned(__builtin_amdgcn_update_dpp(int(keep), int(v), 0x128, 0xf, 0x3, false));
}

// Accumulators are read with explicit v_accvgpr_read so that the compiler
// never copies all 256 of them into VGPRs at once (there is no room).
__device__ __forceinline__ float acc_read(const float& a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
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
    // The tile order (TileOrder: destination by destination with readiness
    // words; XCD-lockstep bands, or grouped rows) is split into queues, one per XCD
    // (workgroups b with b % 8 == x run on XCD x), or a single queue for a grid
    // that is not a multiple of 8.  A queue's workgroups take its first two
    // rounds (one tile each per round) in a fixed order; with tile-claim
    // counters the rest is claimed one tile at a time (the workgroup's own
    // queue first; once it is used up, the queue with the most tiles left), so
    // that XCDs running at a higher clock, or holding fewer tiles, take more
    // and all finish together.  Without counters the workgroups walk their queue a round at a
    // time.
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const bool by_xcd = G % NXCD == 0;
    const int nq = by_xcd ? NXCD : 1;
    const bool claim = a.sched != nullptr;
    TileOrder order(a.tiles_m, a.tiles_n, a.group_m, nq, by_xcd ? a.bands : 0,
                    a.ready ? a.dest_cols : 0, a.part_cols, by_xcd ? a.csplit : 1);
    const int xcd = by_xcd ? bid % NXCD : 0;        // the workgroup's queue
    order.own(xcd);
    auto qlen = [&](int x) { return order.len(x); };
    // logical tile at position i < qlen(x) of queue x
    auto qtile = [&](int x, int i) { return order.logical(x, i); };
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
    // Origin of logical tile l.  n_own: the first output column the tile is
    // responsible for (before the move back), which decides the heads it
    // counts in the readiness words.
    auto tile_origin = [&](int l, int& m0, int& n0, int& n_own) {
        int tm, tn;
        order.coords(l, tm, tn);
        m0 = tm * BM;
        n0 = tn * BN;
        n_own = n0;
        if (!ROWS_CHECKED && m0 + BM > a.M) m0 = a.M - BM;
        if (n0 + BN > a.N) n0 = a.N - BN;
    };

    // ---- global -> LDS: direct loads (buffer_load ... lds) ----------------------
    // Instruction i of wave w fills block b = 4 i + w of a half: lane L brings
    // the chunk stored at slot L % 8 of row r = 8 b + L / 8 of the block, i.e.
    // chunk (L % 8) ^ swz(r) of panel row r; the eight lanes of a row fetch its
    // whole 128-byte segment.  swz(r) = 2 w + (L / 16) % 2 does not depend on
    // the instruction, so every load of a lane uses the same chunk offset.
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.w, (short)0, int(uint32_t(a.N) * uint32_t(K) * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, (short)0, int(uint32_t(a.M) * uint32_t(K) * 2u), 0x00020000);
    // byte sizes are below 2^32 (checked on the host); reads past them return 0
    const uint32_t rowbytes = uint32_t(K) * 2u;
    const int wv = wave;
    const uint32_t lrow = uint32_t(8 * wv + (lane >> 3));
    const uint32_t lchunk = uint32_t((lane & 7) ^ (2 * wv + ((lane >> 4) & 1))) * 16u;
    // this lane's byte offset of K-step 0 of a panel at row origin
    auto panel_offset = [&](int origin) {
        return (uint32_t(origin) + lrow) * rowbytes + lchunk;
    };

    // ---- fragment reads -------------------------------------------------------
    // v_mfma_f32_16x16x32_bf16: lane L holds the A (W) and B (X) operand
    // elements of block row (column) L % 16 and K 8 (L / 16) .. + 7, i.e. chunk
    // 4 s + L / 16 of that row in sub-step s (0, 1) of a K-step; the result in
    // register r of lane L is block row 4 (L / 16) + r of column L % 16.
    // The byte offset of a fragment within a buffer is this lane's part for
    // sub-step s plus a per-block constant, 4096 (blk / 2) + 512 (blk % 2),
    // which rides in the read's immediate offset.
    const int fi = lane & 15;          // block row read; result column (token)
    const int fg = lane >> 4;          // K chunk read; result row group (head dims)
    uint32_t wl[2], xl[2];
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep) {
        const int c = 4 * sstep + fg;
        const int rw_ = wn * 128 + mfma_row(0, fi), rx_ = wm * 128 + mfma_row(0, fi);
        wl[sstep] = uint32_t((rw_ >> 3) * 64 + (rw_ & 7) * 8 + (c ^ lds_swz(rw_))) * 16u;
        xl[sstep] = uint32_t((rx_ >> 3) * 64 + (rx_ & 7) * 8 + (c ^ lds_swz(rx_))) * 16u;
    }
    typedef __attribute__((address_space(3))) uint4 lds_uint4;
    lds_uint4* ring3 = (lds_uint4*)ring;
    const uint32_t ring0 = uint32_t(reinterpret_cast<uintptr_t>(ring3));

    f32x4 acc[8][8];
    // fragments, both 32-deep sub-steps of each block: the eight 16-row W
    // blocks (A operand) of the K-step being multiplied, blocks 0..6 each
    // replaced by the next K-step's block right after its last MFMA and
    // block 7 in two sets, and the eight X blocks (B operand) in two sets,
    // the current K-step's and the next one's (200 VGPRs)
    bf16x8 fa[7][2], fa7[2][2], fb[2][8][2];

    // One MFMA on accumulator (nb, mb); `init`: the tile's first product, with
    // a zero accumulator input (no separate zeroing).
    auto mfma1 = [&](int nb, int mb, const bf16x8& x_, const bf16x8& y_, bool init) __attribute__((always_inline)) {
        if (init)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
                         : "=a"(acc[nb][mb]) : "v"(x_), "v"(y_));
        else
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                         : "+a"(acc[nb][mb]) : "v"(x_), "v"(y_));
    };
    // A fragment read of block blk.  Its result may only be used after a
    // wait that covers it (the compiler does not track it): every use below
    // is an MFMA of a later period, after the closing lgkmcnt(0) wait.
    auto lds_read = [&](bf16x8& dst, uint32_t base, int blk) __attribute__((always_inline)) {
        switch (blk) {
#define QKVX_READ(B) case B: asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) \
                                          : "v"(base), "i"(4096 * ((B) >> 1) + 512 * ((B) & 1))); break;
            QKVX_READ(0) QKVX_READ(1) QKVX_READ(2) QKVX_READ(3)
            QKVX_READ(4) QKVX_READ(5) QKVX_READ(6) QKVX_READ(7)
#undef QKVX_READ
        }
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
    auto load_one = [&](bool is_w, int i, int kidx, uint32_t buf_addr) {
        const bool nx = kidx >= KT;
        const uint32_t g0 = is_w ? (nx ? gw_nxt : gw_cur) : (nx ? gx_nxt : gx_cur);
        const uint32_t kb = uint32_t(nx ? kidx - KT : kidx) * BK * 2u;
        const uint32_t roff = uint32_t(32 * i) * rowbytes;
        lds_uint4* dst = (lds_uint4*)(size_t)(buf_addr + uint32_t((4 * i + wv) * 1024));
        // The buffer's range check covers the VGPR offset but not the SGPR
        // offset.  When rows past M are read (ROWS_CHECKED) the row goes into
        // the VGPR offset so that they read as zeros; otherwise every row read
        // exists and the instruction's row step rides in the SGPR offset with
        // the K offset, which keeps the loop free of address arithmetic.
        const uint32_t voff = ROWS_CHECKED ? g0 + roff : g0;
        const uint32_t soff = ROWS_CHECKED ? kb : roff + kb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_w ? rw : rx,
                                                 (__attribute__((address_space(3))) void*)dst, 16,
                                                 voff, soff, 0, 0);
    };

    // ---- main loop ------------------------------------------------------------
    // The K-steps of this workgroup's tiles form one stream, run in periods.
    // In period g the MFMAs multiply K-step g-1, whose fragments (both 32-deep
    // sub-steps of every W and X block) are in registers, while the fragment
    // reads bring in K-step g and the loads fetch the X half of K-step g+1 and
    // the W half of g+2 into the two buffers K-step g-1 used.  The 128 MFMA
    // slots go row by row: slot j is W block nb = j / 16, X block
    // mb = (j / 2) % 8, sub-step j % 2, so each accumulator takes the two
    // multiply-adds of a K-step back to back (the chip holds a higher clock
    // when an accumulator is written and read again at once: a loop of MFMAs,
    // loads and fragment reads alone ran 15 % faster in this order than with
    // one multiply-add per accumulator in turn, the whole kernel 6-7 %).
    // Fragments: W block nb < 7 is single-buffered, its next K-step read into
    // its registers right after the row's last MFMA (sub-step 0 after slot
    // 16 nb + 14, sub-step 1 after 16 nb + 15); W block 7, whose row ends the
    // period, has two register sets and is read after slots 0 and 1; the X
    // blocks have two sets, the 16 reads of the next one after the even slots
    // 64..98 that carry no other access.  No MFMA waits for a read: every one
    // uses registers filled in the period before, whose end waits for all
    // reads.  Loads go after slots 16 k + 5 and 16 k + 13: the X half in the
    // first half of the period, the W half in the second, and the period's
    // closing wait leaves the W half in flight.  Before the first X read a
    // vmcnt wait makes sure the X half being read has arrived; only a tile's
    // first period actually waits there (see upfront below).
    // pw: the buffer of the W half the period reads (K-step g).  The LDS
    // addresses a period uses (its W and X buffers with both sub-steps'
    // fragment-read bases, and the buffers its loads fill: lx for the X half
    // of g + 1, lw for the W half of g + 2) are carried from the period
    // before, which computes them ahead of its closing barrier: with one wave
    // per SIMD, address arithmetic after the barrier would hold back the
    // period's first MFMAs.
    int pw = 0;
    auto buf_addr = [&](int b) { return ring0 + uint32_t(b) * (BUF_CHUNKS * 16); };
    uint32_t wb = buf_addr(0), xb = buf_addr(1), lx = buf_addr(3), lw = buf_addr(4);
    uint32_t wa0 = wb + wl[0], wa1 = wb + wl[1], xa0 = xb + xl[0], xa1 = xb + xl[1];
    // Closing of a period (or of a tile's up-front part): the next period's
    // addresses, then the waits and the barrier.
    auto advance = [&](bool wait_loads) __attribute__((always_inline)) {
        int pw_n = pw >= 3 ? pw - 3 : pw + 2;            // (pw + 2) % 5
        // opaque to the compiler, so that it derives the addresses from it
        // here (a few scalar operations and four vector adds) instead of
        // keeping every buffer's address in VGPRs through the loop
        asm volatile("" : "+s"(pw_n));
        const int px_n = pw_n == 4 ? 0 : pw_n + 1;
        const int bx1_n = pw_n >= 2 ? pw_n - 2 : pw_n + 3;
        const int bw2_n = pw_n >= 1 ? pw_n - 1 : 4;
        const uint32_t wb_n = buf_addr(pw_n), xb_n = buf_addr(px_n);
        const uint32_t lx_n = buf_addr(bx1_n), lw_n = buf_addr(bw2_n);
        const uint32_t wa0_n = wb_n + wl[0], wa1_n = wb_n + wl[1];
        const uint32_t xa0_n = xb_n + xl[0], xa1_n = xb_n + xl[1];
        if (wait_loads)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(HLOADS), "s"(wb_n),
                         "s"(xb_n), "s"(lx_n), "s"(lw_n), "v"(wa0_n), "v"(wa1_n), "v"(xa0_n),
                         "v"(xa1_n) : "memory");
        else
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::"s"(wb_n), "s"(xb_n), "s"(lx_n),
                         "s"(lw_n), "v"(wa0_n), "v"(wa1_n), "v"(xa0_n), "v"(xa1_n) : "memory");
        pw = pw_n;
        wb = wb_n;
        xb = xb_n;
        lx = lx_n;
        lw = lw_n;
        wa0 = wa0_n;
        wa1 = wa1_n;
        xa0 = xa0_n;
        xa1 = xa1_n;
    };
    // The slot (second half of a period) after which X fragment q = 2 mb + s
    // of the next K-step is read: the even slots 64..98 that are not a row's
    // last two.
    constexpr int XREAD[16] = {64, 66, 68, 70, 72, 74, 76, 80, 82, 84, 86, 88, 90, 92, 96, 98};
    // Period j of the current tile (1 <= j < KT): multiplies K-step j - 1 from
    // register set C (init: the tile's first K-step, zero accumulator inputs)
    // and reads K-step j into set C ^ 1.
    auto period = [&](auto cur, int j, auto first) __attribute__((always_inline)) {
        constexpr int C = decltype(cur)::value;
        constexpr bool init = decltype(first)::value;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                const int mb = p >> 1, sub = p & 1, slot = 16 * nb + p;
                const bf16x8& afr = nb < 7 ? fa[nb][sub] : fa7[C][sub];
                mfma1(nb, mb, afr, fb[C][mb][sub], init && sub == 0);
                if (slot == 0) lds_read(fa7[C ^ 1][0], wa0, 7);
                if (slot == 1) lds_read(fa7[C ^ 1][1], wa1, 7);
                if (nb < 7 && p == 14) lds_read(fa[nb][0], wa0, nb);
                if (nb < 7 && p == 15) lds_read(fa[nb][1], wa1, nb);
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (slot == XREAD[q]) {
                        if (q == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * HLOADS) : "memory");
                        lds_read(fb[C ^ 1][q >> 1][q & 1], (q & 1) ? xa1 : xa0, q >> 1);
                    }
                if (p == 5 || p == 13) {
                    const int v = 2 * nb + (p == 13 ? 1 : 0);
                    if (v < HLOADS) load_one(false, v, j + 1, lx);
                    else load_one(true, v - HLOADS, j + 2, lw);
                }
            }
        }
        advance(true);
    };
    // A tile's up-front part, in place of a period 0: the X half of K-step 1
    // and the W half of K-step 2 go out (held back from the previous tile's
    // end, whose epilogue and tile hand-off use the X buffer as a mailbox),
    // then every fragment of K-step 0 is read into set 0; the closing barrier
    // keeps all waves' reads ahead of period 1's loads into K-step 0's buffers.
    // Period 1's vmcnt wait before its first X read covers the X half of
    // K-step 1 and, as memory operations retire in order, the previous tile's
    // stores.
    auto upfront = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < HLOADS; ++i) load_one(false, i, 1, lx);
#pragma unroll
        for (int i = 0; i < HLOADS; ++i) load_one(true, i, 2, lw);
#pragma unroll
        for (int nb = 0; nb < 7; ++nb) {
            lds_read(fa[nb][0], wa0, nb);
            lds_read(fa[nb][1], wa1, nb);
        }
        lds_read(fa7[0][0], wa0, 7);
        lds_read(fa7[0][1], wa1, 7);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            lds_read(fb[0][mb][0], xa0, mb);
            lds_read(fb[0][mb][1], xa1, mb);
        }
        advance(false);
    };
    // The tile's last K-step, from register set C: no reads, no loads.  The
    // wait drains the W half of the next tile's K-step 1 (its period 1 reads it
    // before any wait).
    auto final_block = [&](auto cur) __attribute__((always_inline)) {
        constexpr int C = decltype(cur)::value;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int p = 0; p < 16; ++p)
                mfma1(nb, p >> 1, nb < 7 ? fa[nb][p & 1] : fa7[C][p & 1], fb[C][p >> 1][p & 1],
                      false);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    // ---- epilogue: one head (128 columns) per wave ----------------------------
    // Accumulator register r of n-block nb in lane group fg holds head dim
    //   e = 32 (nb / 2) + 8 fg + 4 (nb % 2) + r
    // of the token of column fi of m-block mb, tile token
    //   wm * 128 + mfma_row(mb, fi);
    // so for each of H = 0..3 lane group fg holds the eight consecutive dims
    // 32 H + 8 fg .. + 7 (16 bytes of bf16) in n-blocks 2H and 2H+1, n-block
    // nb + 4 holds e + 64 (the rotate-half partner) and registers r, r ^ 1 the
    // interleaved partners.  A token's 128 dims are spread over the four lanes
    // fi + 16 fg, so the RMS reduction is a register sum plus two exchanges,
    // and one store instruction writes, for each of 16 tokens, 64 contiguous
    // bytes from four lanes: 16 requests of 64 bytes, no transposes.
    // Each m-block's 32 values per lane are read from the accumulators once,
    // for the sum of squares, and kept in VGPRs for the outputs.
    //
    // Memory: the norm weights and cos/sin values of (m-block, half) are
    // loaded while the previous half is computed; a Q/K m-block's stores go
    // out after the next block's first loads.  Vector memory operations retire
    // in order, so a wait for loads also waits for every older store: stores
    // are therefore grouped (one group per m-block) and made of whole
    // 128-byte lines.
    // Step (mb, hp), hp = 0, 1, covers dims 32 hp + 8 fg + 0..7 (n-blocks
    // 2 hp, 2 hp + 1) and their partners 64 further on (n-blocks 2 hp + 4,
    // 2 hp + 5).  It needs 4 weight vectors, the same for every m-block (loaded
    // once per tile for both halves), and 2 + 2 cos/sin vectors of its token,
    // loaded one step ahead into the other of two buffers:
    //   W[hp][2 u + c] = w[64 u + 32 hp + 8 fg + 4 c]               (u, c < 2)
    //   rotate-half: C[c] = cs[row][32 hp + 8 fg + 4 c],  S[c] at + 64
    //   interleaved: C[u] = cs[row][16 (hp + 2 u) + 4 fg], S[u] at + 64
    f32x4 Wf[2][4], Cb[2][2], Sb[2][2];
    auto load_weights = [&](const float* nw) {
#pragma unroll
        for (int hp = 0; hp < 2; ++hp)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Wf[hp][i] = *reinterpret_cast<const f32x4*>(nw + 64 * (i >> 1) + 32 * hp +
                                                            8 * fg + 4 * (i & 1));
    };
    auto load_tables = [&](int row, int hp, int buf) {
        const float* csr = a.cs + int64_t(row) * 128;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int off = ROPE_IL ? 16 * (hp + 2 * i) + 4 * fg : 32 * hp + 8 * fg + 4 * i;
            Cb[buf][i] = *reinterpret_cast<const f32x4*>(csr + off);
            Sb[buf][i] = *reinterpret_cast<const f32x4*>(csr + 64 + off);
        }
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
        const int m_tile = m0 + wm * 128 + mfma_row(mb, fi);
        in_range = m_tile < a.M;
        const int m = in_range ? m_tile : a.M - 1;
        uint32_t bidx, s;
        a.div_s.divmod(uint32_t(m), bidx, s);
        return make_int2(int(bidx), a.row0 + int(s));   // batch, sequence row == position
    };
    // Stores of one m-block: out[H] holds dims 32 H + 8 fg .. + 7 of this
    // lane's token, at byte 64 H + 16 fg of its 256-byte head vector.  Lanes
    // fi and fi ^ 8 (tokens 16 apart) trade one piece of each pair H = 2P,
    // 2P + 1, so that every store instruction writes whole 128-byte lines:
    // the first store of a pair writes both halves of line P for the tokens of
    // lanes fi < 8, the second for those of lanes fi >= 8.  Written as 64-byte
    // halves from two instructions, nontemporal lines leave the L2 as two
    // partial writes.
    // off: the token row's element offset from dbase.  Called with all 64
    // lanes active (wave-uniform control flow only): the DPP moves read the
    // partner lane's registers, and out-of-range tokens are skipped at the
    // stores, after the trade.
    auto store_block = [&](int64_t off, bool in_range, const uint4* out) {
        const bool low = fi < 8;
        const uint64_t own = uint64_t(off);
        const int64_t other = int64_t(uint64_t(swap8(uint32_t(own))) |
                                      (uint64_t(swap8(uint32_t(own >> 32))) << 32));
        const bool pin = swap8(in_range ? 1u : 0u) != 0u;
        // first store of a pair: low lanes their own token's dims 0..31 of the
        // line, high lanes their partner's dims 32..63; second store: the
        // other way round (line P is 64 P further on: an immediate offset)
        uint16_t* pa = dbase + (low ? off : other + 32) + 8 * fg;
        uint16_t* pb = dbase + (low ? other : off + 32) + 8 * fg;
        const bool ina = low ? in_range : pin, inb = low ? pin : in_range;
#pragma unroll
        for (int P = 0; P < 2; ++P) {
            const uint4 x0 = out[2 * P], x1 = out[2 * P + 1];
            uint4 a, b;
            a.x = take_hi(x0.x, x1.x); a.y = take_hi(x0.y, x1.y);
            a.z = take_hi(x0.z, x1.z); a.w = take_hi(x0.w, x1.w);
            b.x = take_lo(x1.x, x0.x); b.y = take_lo(x1.y, x0.y);
            b.z = take_lo(x1.z, x0.z); b.w = take_lo(x1.w, x0.w);
            if (ina) store_stream(pa + 64 * P, a);
            if (inb) store_stream(pb + 64 * P, b);
        }
    };
    // eight consecutive dims (n-blocks 2H and 2H+1) -> one 16-byte piece
    auto pack8 = [&](const float (&v)[2][4]) {
        uint4 pk;
        pk.x = bf16_pair(v[0][0], v[0][1]);
        pk.y = bf16_pair(v[0][2], v[0][3]);
        pk.z = bf16_pair(v[1][0], v[1][1]);
        pk.w = bf16_pair(v[1][2], v[1][3]);
        return pk;
    };

    if (p == 2) {
        // V: rounding and placement only
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            bool in_range;
            const auto br = token_row(mb, in_range);
            const int64_t off = int64_t(br.x) * a.stride_b + int64_t(br.y) * a.stride_s;
            uint4 out[4];
#pragma unroll
            for (int H = 0; H < 4; ++H) {
                float v[2][4];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[t][r] = acc_read(acc[2 * H + t][mb][r]);
                out[H] = pack8(v);
            }
            store_block(off, in_range, out);
        }
        __builtin_amdgcn_sched_barrier(0);
        return;
    }

    // The weights and step 0 (m-block 0, half 0) of the table go out first:
    // no ring loads are in flight here (the last K-step drained them and the
    // next tile's first loads go out after the epilogue), so they wait for
    // nothing else, and the m-block 0 sum of squares overlaps their latency.
    int rows[8], bats[8];
    bool in_range[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const auto br = token_row(mb, in_range[mb]);
        bats[mb] = br.x;
        rows[mb] = br.y;
    }
    auto load_step = [&](int mb, int hp, int buf) { load_tables(rows[mb], hp, buf); };
    load_weights(p == 0 ? a.wq : a.wk);
    load_step(0, 0, 0);

#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        // RMSNorm over the head's 128 values: 32 here, 96 in lanes ^ 16, ^ 32;
        // the block's 32 values are read from the accumulators once
        float y[8][4];
        float ss = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                y[nb][r] = acc_read(acc[nb][mb][r]);
                ss += y[nb][r] * y[nb][r];
            }
        ss = sum_lane_groups(ss);
        const float inv = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
        uint4 out[4];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            const int cur = (2 * mb + hp) & 1;
            if (2 * mb + hp < 15) load_step(hp == 0 ? mb : mb + 1, hp ^ 1, cur ^ 1);
            // lo[t][r]: dim 32 hp + 8 fg + 4 t + r; hi: the same + 64
            float lo[2][4], hi[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lo[t][r] = y[2 * hp + t][r];
                    hi[t][r] = y[2 * hp + 4 + t][r];
                }
            if (ROPE_IL) {
                // pairs (2i, 2i+1) = registers (r, r+1), r = 0, 2, of each
                // n-block; run u (lo, hi) rotates by table columns
                // 16 (hp + 2 u) + 4 fg + 2 t + r / 2
                auto rotate_run = [&](float (&v)[2][4], const int u) __attribute__((always_inline)) {
                    const f32x4 cv = Cb[cur][u], sv = Sb[cur][u];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4 wt = Wf[hp][2 * u + t];
#pragma unroll
                        for (int gp = 0; gp < 2; ++gp) {
                            const float z0 = v[t][2 * gp] * (inv * wt[2 * gp]);
                            const float z1 = v[t][2 * gp + 1] * (inv * wt[2 * gp + 1]);
                            const float c = cv[2 * t + gp], sn = sv[2 * t + gp];
                            v[t][2 * gp] = z0 * c - z1 * sn;
                            v[t][2 * gp + 1] = z1 * c + z0 * sn;
                        }
                    }
                };
                rotate_run(lo, 0);
                rotate_run(hi, 1);
            } else {
                // rotate-half: lo and hi hold dims e and e + 64, angle column
                // 32 hp + 8 fg + 4 t + r
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const f32x4 wl_ = Wf[hp][t], wh_ = Wf[hp][2 + t];
                    const f32x4 cv = Cb[cur][t], sv = Sb[cur][t];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float zl = lo[t][r] * (inv * wl_[r]);
                        const float zh = hi[t][r] * (inv * wh_[r]);
                        lo[t][r] = zl * cv[r] - zh * sv[r];
                        hi[t][r] = zh * cv[r] + zl * sv[r];
                    }
                }
            }
            out[hp] = pack8(lo);
            out[hp + 2] = pack8(hi);
            __builtin_amdgcn_sched_barrier(0);
        }
        // this block's stores go out after the next block's first loads
        store_block(int64_t(bats[mb]) * a.stride_b + int64_t(rows[mb]) * a.stride_s, in_range[mb],
                    out);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

    // claim state (thread 0 only): the queue counter being drawn from
    int cvict = xcd;

    // prologue: W and X halves of K-step 0 and the W half of K-step 1 (the
    // first tile's up-front part loads the X half of K-step 1 and the W half
    // of K-step 2)
#pragma unroll
    for (int i = 0; i < HLOADS; ++i) load_one(true, i, 0, buf_addr(0));
#pragma unroll
    for (int i = 0; i < HLOADS; ++i) load_one(false, i, 0, buf_addr(1));
#pragma unroll
    for (int i = 0; i < HLOADS; ++i) load_one(true, i, 1, buf_addr(2));
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    typedef std::integral_constant<int, 0> set0;
    typedef std::integral_constant<int, 1> set1;
    typedef std::integral_constant<bool, true> first_step;
    typedef std::integral_constant<bool, false> later_step;
    for (;;) {
        upfront();
        // period 1 (the tile's first products), periods 2 .. KT-1 in pairs
        // (set 1, set 0), then the last K-step from set 1: K = 128 * heads,
        // so KT = K / 64 is even and at least 2, and every tile ends on the
        // same code (no join of two code paths with live accumulators)
        period(set0(), 1, first_step());
        for (int j = 2; j < KT; j += 2) {
            period(set1(), j, later_step());
            period(set0(), j + 1, later_step());
        }
        final_block(set1());
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
                    // This queue is used up: read every queue's counter at once
                    // (independent loads, one round trip) and claim from the one
                    // with the most tiles left; none left ends the workgroup's
                    // claims.  Counters only grow, so a count read here never
                    // overstates what is left, and each claim moves one on.
                    int best = -1, most = 0;
                    unsigned int seen[NXCD];
#pragma unroll
                    for (int q = 0; q < NXCD; ++q)
                        if (q < nq)
                            seen[q] = __hip_atomic_load(a.sched + q, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                    for (int q = 0; q < NXCD; ++q)
                        if (q < nq) {
                            const int left = qlen(q) - (2 * stride + int(seen[q]));
                            if (left > most) {
                                most = left;
                                best = q;
                            }
                        }
                    if (best < 0) break;
                    cvict = best;
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

namespace {
__global__ __launch_bounds__(64) void clear_words_kernel(unsigned int* p, int n) {
    for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}
}  // namespace

hipError_t scratch_address(unsigned int** out) {
    static std::mutex mu;
    static unsigned int* ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptr[dev] = static_cast<unsigned int*>(p);
    }
    *out = ptr[dev];
    return hipSuccess;
}

hipError_t launch_clear_words(unsigned int* p, int n, hipStream_t stream) {
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(64), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs& a_in, hipStream_t stream) {
    FusedArgs a = a_in;
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    a.group_m = GROUP_M;
    a.div_s = FastDiv(uint32_t(a.s_local));
    const int tiles = a.tiles_m * a.tiles_n;
    // with readiness words one CU per XCD stays free, so that wait kernels on
    // other streams always find room while this grid runs
    const int all_cus = device_cus();
    const int cus = a.ready && all_cus > 2 * NXCD ? all_cus - NXCD : all_cus;
    const int grid = tiles < cus ? tiles : cus;
    a.bands = lockstep_bands(a.tiles_m, a.K, BM, grid, NXCD);
    a.csplit = lockstep_csplit(a.tiles_m, a.ready && a.dest_cols > 0 ? 3 * a.dest_cols : a.tiles_n,
                               a.bands, grid, NXCD);
    auto kernel = a.M < BM ? (a.rope_interleaved ? fused_qkv_kernel<true, true>
                                                 : fused_qkv_kernel<true, false>)
                           : (a.rope_interleaved ? fused_qkv_kernel<false, true>
                                                 : fused_qkv_kernel<false, false>);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qkvx
