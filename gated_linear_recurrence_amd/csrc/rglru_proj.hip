// Dense projections around the recurrent block's path, for gfx950 (CDNA4).
//
// The page "Gemma 詳解：RecurrentGemma 架構" (section "含遞迴區塊的殘差區塊" and the module
// printout) puts three Linear layers with bias around the path: linear_x and linear_y take the
// block input (width 2560) to the two branches (width 2560) in parallel, and linear_out takes
// the product of the branches back to the block width.  A Linear layer with weight W [out][in]
// computes
//
//   C[m][n] = bias[n] + sum_k A[m][k] W[n][k]
//
// Here: bf16 operands, fp32 accumulation on MFMA, bf16 results (round to nearest even).  The
// two branch projections run as one GEMM with N = 2 D: output tiles left of D read linear_x's
// weight and write x, the others read linear_y's weight and write y (up to three such output
// segments; the attention block's q, k and v are another use).
//
// Workgroup tile 256 x 256, four waves of 128 x 128 (4 x 4 tiles of v_mfma_f32_32x32x16_bf16,
// 256 fp32 accumulators per lane, in AGPRs).  K advances in steps of 64 through two LDS stages
// filled by buffer loads with the LDS bit (16 bytes per lane, straight into LDS), one k-step
// ahead of the MFMAs.  A k-step reads whole 128-byte lines of its 512 tile rows; with 32-byte
// k-steps each line was fetched twice (the L1 cannot keep 512 lines between the halves).
#include <algorithm>
#include <type_traits>

#include "rglru_device.h"
#include "rglru_internal.h"
#include "rglru_lds_copy.h"

namespace rglru {
namespace {

typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

constexpr int kBM = 256;                    // tile rows (M)
constexpr int kBN = 256;                    // tile columns (N)
constexpr int kBK = 64;                     // K per stage
constexpr int kSkinnyRows = 64;             // at most this many rows: skinny_gemm_kernel (taken
                                            // when the caller gives no partial-sum space)
constexpr int kRowsMax = 4;                 // at most this many rows: gemv_rows_kernel
constexpr int kThreads = 256;               // 4 waves, 2 x 2 over the tile
constexpr int kChunks = kBK / 8;            // 16-byte chunks per tile row
constexpr int kRowBytes = kBK * 2;
constexpr int kTileBytes = kBM * kRowBytes;             // one operand, one stage: 32 KB
constexpr int kCopiesPerWave = kTileBytes / 1024 / 4;   // 1 KB copies per wave, operand, stage
constexpr int kGroupM = 8;                  // tile rows per group of the tile order
static_assert(kBM == kBN, "both operands share the copy and fragment helpers");
static_assert(kChunks == 8 && kCopiesPerWave == 8, "the swizzle and copies are for 128-byte rows");

// Position of 16-byte chunk c of tile row r inside its 128-byte row.  A fragment read has 16
// lanes on 16 consecutive rows at one chunk index; chunk c of row r goes to c ^ f(r) with
// f(r) = (r ^ (r / 8)) % 8, which puts the 16 reads in 16 distinct 16-byte bank groups of a
// 256-byte bank line (and any 8 consecutive rows in distinct groups of a 128-byte line).
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

// Half of one operand's copies of k-step kt into an LDS stage (this wave's copies 4 h .. 4 h + 3
// of its 8).  Lane l of copy q fills LDS chunk p = 64 q + l of the stage (row p / 8, position
// p % 8), so the global side reads the chunk that belongs there (the swizzle is its own
// inverse).  Tile row r is global row min(r, rows - 1) relative to the resource base: rows past
// a ragged M repeat the last row and their results are never stored.
__device__ __forceinline__ void copy_half(const u32x4& rs, uint16_t* lds, int h, int wv,
                                          int lane, int K, int rows, int kt, int row_off = 0) {
    int off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int p = (wv * kCopiesPerWave + 4 * h + j) * 64 + lane;
        const int r = p / kChunks;
        const int c = chunk_pos(r, p % kChunks);
        off[j] = (min(r, rows - 1) - row_off) * K * 2 + kt * kRowBytes + 16 * c;
    }
    copy4(rs, lds_address(lds + (wv * kCopiesPerWave + 4 * h) * 512), off);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// A or B fragment of the 32-row tile starting at row r0, K sub-step s (16 k): lane l supplies
// row r0 + l % 32 and k = 16 s + 8 (l / 32) .. + 7.
__device__ __forceinline__ bf16x8 frag(const uint16_t* lds, int r0, int lane, int s) {
    const int r = r0 + (lane & 31);
    const int c = 2 * s + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(lds + r * kBK + 8 * chunk_pos(r, c));
}

// The lane's fragments of one K sub-step: 4 A tiles (rows 128 wm + 32 i) and 4 weight tiles
// (rows 128 wn + 32 j).
__device__ __forceinline__ void load_frags(const uint16_t* sa, const uint16_t* sb, int s, int wm,
                                          int wn, int lane, bf16x8 (&a)[4], bf16x8 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag(sa, 128 * wm + 32 * i, lane, s);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = frag(sb, 128 * wn + 32 * j, lane, s);
}

// 16 MFMAs of one K sub-step.  Weight rows are the MFMA's A operand: the result tile is C^T,
// so each lane ends up with 4 consecutive output columns per register group (8-byte stores).
__device__ __forceinline__ void mma(const bf16x8 (&a)[4], const bf16x8 (&b)[4],
                                    f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
}

// The 16 MFMAs of one K sub-step (fragments a, b) with the 8 fragment loads of the next
// sub-step (from stage na/nb, sub-step ns, into a2/b2) placed one after each of the first 8
// MFMAs, and an optional extra unit of work (the stage refill) after MFMAs 8..11.  The order is
// pinned (sched_barrier): left free, the compiler moved the loads next to their first use and
// waited for them there.
template <typename Extra>
__device__ __forceinline__ void mma_pipe(const bf16x8 (&a)[4], const bf16x8 (&b)[4],
                                         f32x16 (&acc)[4][4], const uint16_t* na,
                                         const uint16_t* nb, int ns, int wm, int wn, int lane,
                                         bf16x8 (&a2)[4], bf16x8 (&b2)[4], Extra&& extra) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int i = u >> 2, j = u & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
        if (u < 4) a2[u] = frag(na, 128 * wm + 32 * u, lane, ns);
        else if (u < 8) b2[u - 4] = frag(nb, 128 * wn + 32 * (u - 4), lane, ns);
        else if (u < 12) extra(u - 8);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Workgroup -> output tile.  Workgroups go to the 8 XCDs round-robin; each XCD is given one
// contiguous range of the tile order, and the tile order walks groups of kGroupM tile rows
// column by column, so the ~32 workgroups an XCD runs at once share A rows and W rows in its L2.
__device__ __forceinline__ void tile_of(int bid, int ntm, int ntn, int& tm, int& tn) {
    const int tiles = ntm * ntn;
    const int L = (tiles & 7) == 0 ? (bid & 7) * (tiles >> 3) + (bid >> 3) : bid;
    const int per_group = kGroupM * ntn;
    const int grp = L / per_group;
    const int first = grp * kGroupM;
    const int gm = min(ntm - first, kGroupM);
    const int r = L - grp * per_group;
    tm = first + r % gm;
    tn = r / gm;
}

// kGated (no K split; two segments of equal width, gate and up): a tile takes 128 features of
// both, the gate rows in tile columns 0..127 and the up rows of the same features in 128..255
// (waves 0 and 1 copy the gate rows, waves 2 and 3 the up rows), so waves (wm, 0) and (wm, 1)
// hold gate and up of the same outputs in the same registers; the up half hands its rounded
// values over through LDS and the gate half writes gelu_tanh(gate) * up, rounded as the
// separate gating step rounds it.
template <bool kSplitK, bool kGated = false>
__global__ void __launch_bounds__(kThreads, 1) proj_gemm_kernel(ProjGemmArgs g) {
    static_assert(!(kSplitK && kGated), "the gating of split sums runs in the reduction");
    __shared__ __attribute__((aligned(16))) uint16_t a0[kBM * kBK], a1[kBM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t b0[kBN * kBK], b1[kBN * kBK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (the copies' LDS base)
    const int wm = wv >> 1, wn = wv & 1;
    int tm, tn;
    // with K split, blocks tiles * ks .. tiles * (ks + 1) - 1 take split ks of every tile; with
    // a batch, each item's blocks follow the previous item's
    const int tiles = g.ntm * g.ntn;
    const int per_item = tiles * (kSplitK ? g.ksplit : 1);
    const int bi = g.batch > 1 ? __builtin_amdgcn_readfirstlane((int)blockIdx.x / per_item) : 0;
    const int bloc = (int)blockIdx.x - bi * per_item;
    const int ks = kSplitK ? __builtin_amdgcn_readfirstlane(bloc / tiles) : 0;
    tile_of(bloc - ks * tiles, g.ntm, g.ntn, tm, tn);
    // the divisions above run on the vector unit; the tile is uniform, and the buffer resources
    // built from it must sit in scalar registers
    const int m0 = __builtin_amdgcn_readfirstlane(tm) * kBM;
    // gated: the tile's features are n0 .. n0 + 127 of both segments
    const int n0 = __builtin_amdgcn_readfirstlane(tn) * (kGated ? kBN / 2 : kBN);
    // output segment of this tile (segment widths are multiples of the tile width)
    const int seg = kGated ? 0 : (n0 < g.Nw[0] ? 0 : (n0 < g.Nw[0] + g.Nw[1] ? 1 : 2));
    const int nl0 = kGated ? n0 : n0 - (seg > 0 ? g.Nw[0] : 0) - (seg > 1 ? g.Nw[1] : 0);
    // gated: waves 2 and 3 copy tile rows 128..255, the up rows of the same features
    const int wseg = kGated && wv >= 2 ? 1 : seg, wrow_off = kGated && wv >= 2 ? kBN / 2 : 0;
    const int K = g.K;                            // row pitch of A and W
    const int Ks = kSplitK ? K / g.ksplit : K;   // this block's share of K
    const int k0 = ks * Ks;
    const int rows = min(g.M - m0, kBM);
    const uint16_t* A = static_cast<const uint16_t*>(g.A) + (size_t)bi * g.bsA + (size_t)m0 * K + k0;
    const uint16_t* W = static_cast<const uint16_t*>(g.W[wseg]) + (size_t)bi * g.bsW + (size_t)nl0 * K + k0;
    // (the ranges run k0 elements past the last row's share; no access reaches that far)
    const u32x4 ra = rsrc_words(A, (uint32_t)(rows * K * 2));
    const u32x4 rb = rsrc_words(W, (uint32_t)(kBN * K * 2));
    const int KT = Ks / kBK;                      // even, >= 2

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    constexpr int kPerStep = 2 * kCopiesPerWave;  // copies per wave per k-step
    guard_vmem_sgprs(ra, rb);
    copy_half(ra, a0, 0, wv, lane, K, rows, 0);
    copy_half(ra, a0, 1, wv, lane, K, rows, 0);
    copy_half(rb, b0, 0, wv, lane, K, kBN, 0, wrow_off);
    copy_half(rb, b0, 1, wv, lane, K, kBN, 0, wrow_off);
    copy_half(ra, a1, 0, wv, lane, K, rows, 1);
    copy_half(ra, a1, 1, wv, lane, K, rows, 1);
    copy_half(rb, b1, 0, wv, lane, K, kBN, 1, wrow_off);
    copy_half(rb, b1, 1, wv, lane, K, kBN, 1, wrow_off);
    wait_vmcnt<kPerStep>();
    lds_sync();
    bf16x8 fa[4], fb[4];                           // fragments of the current k-step's sub-step 0
    load_frags(a0, b0, 0, wm, wn, lane, fa, fb);

    // One k-step of four K sub-steps, fragments ping-ponging between two register sets (each
    // sub-step's loads arrive under the previous sub-step's MFMAs).  After the third sub-step
    // this wave waits for its copies of the next stage and meets the other waves: the next
    // stage is then complete, and nobody reads the current one any more (its last fragments
    // are in registers), so its refill (k-step kt + 2) is issued between the fourth sub-step's
    // MFMAs, after the next k-step's first fragments.  F (compile time): kRefill | kNext.
    // A runtime branch there made the compiler's LDS wait counts fall back to the shorter path.
    constexpr int kRefill = 1, kNext = 2;
    auto step = [&](auto flags, int kt, uint16_t* ca, uint16_t* cb, const uint16_t* xa,
                    const uint16_t* xb) {
        constexpr int F = decltype(flags)::value;
        auto none = [](int) {};
        bf16x8 ga[4], gb[4];
        __builtin_amdgcn_sched_barrier(0);
        mma_pipe(fa, fb, acc, ca, cb, 1, wm, wn, lane, ga, gb, none);
        mma_pipe(ga, gb, acc, ca, cb, 2, wm, wn, lane, fa, fb, none);
        mma_pipe(fa, fb, acc, ca, cb, 3, wm, wn, lane, ga, gb, none);
        if constexpr ((F & kNext) != 0) {
            wait_vmcnt<0>();
            lds_sync();
            __builtin_amdgcn_sched_barrier(0);
            auto refill = [&](int h) {
                if constexpr ((F & kRefill) != 0) {
                    if (h < 2) copy_half(ra, ca, h, wv, lane, K, rows, kt + 2);
                    else copy_half(rb, cb, h - 2, wv, lane, K, kBN, kt + 2, wrow_off);
                }
            };
            mma_pipe(ga, gb, acc, xa, xb, 0, wm, wn, lane, fa, fb, refill);
        } else {
            mma(ga, gb, acc);
        }
    };
    using All = std::integral_constant<int, kRefill | kNext>;
    using NextOnly = std::integral_constant<int, kNext>;
    using Fin = std::integral_constant<int, 0>;
    // The stage of k-step kt is kt % 2.  Step 0 runs before the loop, so the loop's first step
    // reads stage 1 (with stage 0 read right after the loop header the compiler's wait
    // accounting merged the paths into the loop conservatively).  The loop runs k-steps
    // 1 .. KT - 4, each of which refills and has a next; the last three follow it.
    if (KT == 2) {
        step(NextOnly{}, 0, a0, b0, a1, b1);
        step(Fin{}, 1, a1, b1, a0, b0);
    } else {
        step(All{}, 0, a0, b0, a1, b1);
        for (int kt = 1; kt < KT - 3; kt += 2) {
            step(All{}, kt, a1, b1, a0, b0);
            step(All{}, kt + 1, a0, b0, a1, b1);
        }
        step(All{}, KT - 3, a1, b1, a0, b0);
        step(NextOnly{}, KT - 2, a0, b0, a1, b1);
        step(Fin{}, KT - 1, a1, b1, a0, b0);
    }

    // acc[i][j] is the transposed 32 x 32 tile: lane l holds output row 32 i + l % 32 and, in
    // registers 4 q .. 4 q + 3, output columns 32 j + 8 q + 4 (l / 32) + 0..3.  Buffer ranges end at
    // the last valid row, so stores of rows past a ragged M are dropped.
    const int ncol = 128 * wn + 4 * (lane >> 5);
    const int mrow = 128 * wm + (lane & 31);
    if constexpr (kSplitK) {
        // fp32 partial sums of this split, [ks][M][Ntot], four columns per 16-byte store
        const int ntot = g.ntn * kBN;
        float* P = g.part + (size_t)bi * g.ksplit * g.M * ntot + ((size_t)ks * g.M + m0) * ntot + n0;
        const __amdgpu_buffer_rsrc_t rp = make_rsrc_n(P, (uint32_t)(rows * ntot * 4));
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x16& t = acc[i][j];
                    const f32x4 v = {t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
                    const int off = ((mrow + 32 * i) * ntot + ncol + 32 * j + 8 * q) * 4;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp, off,
                                                           0, 0);
                }
        return;
    }
    if constexpr (kGated) {
        // gate (wn = 0) and up (wn = 1) of features n0 + 32 j + 8 q + 4 (l / 32) + 0..3, rounded
        // with their biases; up through LDS (stage memory, free once every wave is past its last
        // MFMA operands: 32 KB per up wave)
        const uint16_t* bias = static_cast<const uint16_t*>(g.b[wn]);
        u32x2* const xb = reinterpret_cast<u32x2*>(wm ? a1 : a0);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = n0 + 4 * (lane >> 5) + 32 * j + 8 * q;
                const uint2 bw = bias ? *reinterpret_cast<const uint2*>(bias + f) : make_uint2(0u, 0u);
                const float bv[4] = {bf_lo(bw.x), bf_hi(bw.x), bf_lo(bw.y), bf_hi(bw.y)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x16& t = acc[i][j];
                    const u32x2 v = {pack2bf(t[4 * q] + bv[0], t[4 * q + 1] + bv[1]),
                                     pack2bf(t[4 * q + 2] + bv[2], t[4 * q + 3] + bv[3])};
                    const int slot = ((i * 4 + j) * 4 + q) * 64 + lane;
                    if (wn == 1) xb[slot] = v;
                    else acc[i][j][4 * q] = __uint_as_float(v[0]), acc[i][j][4 * q + 1] = __uint_as_float(v[1]);
                }
            }
        __syncthreads();
        if (wn == 1) return;
        const int ldc = g.Nw[0];
        uint16_t* C = static_cast<uint16_t*>(g.C[0]) + (size_t)m0 * ldc + n0;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc_n(C, (uint32_t)(rows * ldc * 2));
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x2 gt = {__float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1])};
                    const u32x2 up = xb[((i * 4 + j) * 4 + q) * 64 + lane];
                    const u32x2 v = {pack2bf(gelu_fast(bf_lo(gt[0])) * bf_lo(up[0]), gelu_fast(bf_hi(gt[0])) * bf_hi(up[0])),
                                     pack2bf(gelu_fast(bf_lo(gt[1])) * bf_lo(up[1]), gelu_fast(bf_hi(gt[1])) * bf_hi(up[1]))};
                    const int off = ((mrow + 32 * i) * ldc + 4 * (lane >> 5) + 32 * j + 8 * q) * 2;
                    __builtin_amdgcn_raw_buffer_store_b64(v, rc, off, 0, 0);
                }
        return;
    }
    // bias, round, store
    const uint16_t* bias = g.b[seg] ? static_cast<const uint16_t*>(g.b[seg]) + (size_t)bi * g.bsb : nullptr;
    const int ldc = g.Nw[seg];
    uint16_t* C = static_cast<uint16_t*>(g.C[seg]) + (size_t)bi * g.bsC + (size_t)m0 * ldc + nl0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc_n(C, (uint32_t)(rows * ldc * 2));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint2 bw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bw[q] = bias ? *reinterpret_cast<const uint2*>(bias + nl0 + ncol + 32 * j + 8 * q)
                         : make_uint2(0u, 0u);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = ncol + 32 * j + 8 * q;
            const float bv[4] = {bf_lo(bw[q].x), bf_hi(bw[q].x), bf_lo(bw[q].y), bf_hi(bw[q].y)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x16& t = acc[i][j];
                const u32x2 v = {pack2bf(t[4 * q] + bv[0], t[4 * q + 1] + bv[1]),
                                 pack2bf(t[4 * q + 2] + bv[2], t[4 * q + 3] + bv[3])};
                const int off = ((mrow + 32 * i) * ldc + n) * 2;
                __builtin_amdgcn_raw_buffer_store_b64(v, rc, off, 0, 0);
            }
        }
    }
}

// C = bias + the sum of the K splits' partials, in split order; eight columns per thread (a
// segment's columns are a multiple of the tile width, so eight never straddle two segments).
// Sum of eight columns' partials in split order (as one GEMM adds its k-steps).
__device__ __forceinline__ void sum_splits(const ProjGemmArgs& g, const float* part, int m, int ntot,
                                           int n, float (&acc)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    for (int s = 0; s < g.ksplit; ++s) {
        const float4* p = reinterpret_cast<const float4*>(part + ((size_t)s * g.M + m) * ntot + n);
        const float4 x = p[0], y = p[1];
        acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
        acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
    }
}
__device__ __forceinline__ void bias8(const uint16_t* bias, int n, float (&v)[8]) {
    if (bias) {
        const uint4 b = *reinterpret_cast<const uint4*>(bias + n);
        const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = bf_lo(w[k]);
            v[2 * k + 1] = bf_hi(w[k]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.0f;
    }
}

__global__ void __launch_bounds__(256) proj_splitk_reduce_kernel(ProjGemmArgs g) {
    const int ntot = g.ntn * kBN, n8 = (g.gated ? g.Nw[0] : ntot) / 8;
    const size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int nb = g.batch > 1 ? g.batch : 1;
    if (i0 >= (size_t)nb * g.M * n8) return;
    const size_t bi = i0 / ((size_t)g.M * n8), i = i0 - bi * ((size_t)g.M * n8);
    const int m = (int)(i / n8), n = (int)(i % n8) * 8;
    if (g.gated) {
        // gate columns n.., up columns Nw[0] + n..: each rounded with its bias, then the gating
        // step's gelu_tanh(gate) * up, rounded
        float ag[8], au[8], vg[8], vu[8];
        sum_splits(g, g.part, m, ntot, n, ag);
        sum_splits(g, g.part, m, ntot, g.Nw[0] + n, au);
        bias8(static_cast<const uint16_t*>(g.b[0]), n, vg);
        bias8(static_cast<const uint16_t*>(g.b[1]), n, vu);
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t gw = pack2bf(ag[2 * k] + vg[2 * k], ag[2 * k + 1] + vg[2 * k + 1]);
            const uint32_t uw = pack2bf(au[2 * k] + vu[2 * k], au[2 * k + 1] + vu[2 * k + 1]);
            o[k] = pack2bf(gelu_fast(bf_lo(gw)) * bf_lo(uw), gelu_fast(bf_hi(gw)) * bf_hi(uw));
        }
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g.C[0]) + (size_t)m * g.Nw[0] + n) =
            make_uint4(o[0], o[1], o[2], o[3]);
        return;
    }
    const int seg = n < g.Nw[0] ? 0 : (n < g.Nw[0] + g.Nw[1] ? 1 : 2);
    const int nl = n - (seg > 0 ? g.Nw[0] : 0) - (seg > 1 ? g.Nw[1] : 0);
    float v[8];
    const uint16_t* bias = g.b[seg] ? static_cast<const uint16_t*>(g.b[seg]) + bi * g.bsb : nullptr;
    const float* part = g.part + bi * g.ksplit * g.M * ntot;
    if (bias) {
        const uint4 b = *reinterpret_cast<const uint4*>(bias + nl);
        const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = bf_lo(w[k]);
            v[2 * k + 1] = bf_hi(w[k]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.0f;
    }
    // the partials are added in split order (as one GEMM adds its k-steps), then the bias
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s = 0; s < g.ksplit; ++s) {
        const float4* p = reinterpret_cast<const float4*>(part + ((size_t)s * g.M + m) * ntot + n);
        const float4 x = p[0], y = p[1];
        acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
        acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
    }
    if (g.c_f32) {
        float4* Cf = reinterpret_cast<float4*>(static_cast<float*>(g.C[seg]) + bi * g.bsC + (size_t)m * g.Nw[seg] + nl);
        Cf[0] = make_float4(acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]);
        Cf[1] = make_float4(acc[4] + v[4], acc[5] + v[5], acc[6] + v[6], acc[7] + v[7]);
        return;
    }
    uint16_t* C = static_cast<uint16_t*>(g.C[seg]) + bi * g.bsC + (size_t)m * g.Nw[seg] + nl;
    *reinterpret_cast<uint4*>(C) = make_uint4(pack2bf(acc[0] + v[0], acc[1] + v[1]),
                                              pack2bf(acc[2] + v[2], acc[3] + v[3]),
                                              pack2bf(acc[4] + v[4], acc[5] + v[5]),
                                              pack2bf(acc[6] + v[6], acc[7] + v[7]));
}

// The residual layer's add-and-norm fused into the split-K sum (rows_epilogue): one workgroup
// of 256 threads per row of at most 8192 columns, eight columns per thread and step.
// C = R + (bias + the split partials in split order), each rounding as the separate GEMM, sum
// and add_rmsnorm steps make it; with norm_out also the row's RMSNorm(C) * norm_g from the
// rounded C in fp32 (sum of squares per thread, then per wave, then the four waves in order).
constexpr int kRowsMaxChunks = 4;    // 8-column chunks per thread
__device__ __forceinline__ float row_wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__global__ void __launch_bounds__(256) proj_splitk_rows_kernel(ProjGemmArgs g) {
    __shared__ float wsum[4];
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int ntot = g.Nw[0], nch = ntot / 8;
    const uint16_t* bias = static_cast<const uint16_t*>(g.b[0]);
    const uint16_t* R = static_cast<const uint16_t*>(g.R);
    uint16_t* C = static_cast<uint16_t*>(g.C[0]) + (size_t)row * ntot;
    uint4 hv[kRowsMaxChunks];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsMaxChunks; ++i) {
        const int c = tid + 256 * i;
        if (c >= nch) continue;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int s = 0; s < g.ksplit; ++s) {
            const float4* p = reinterpret_cast<const float4*>(g.part + ((size_t)s * g.M + row) * ntot + 8 * c);
            const float4 x = p[0], y = p[1];
            acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
            acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
        }
        float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (bias) {
            const uint4 b = *reinterpret_cast<const uint4*>(bias + 8 * c);
            const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[2 * k] = bf_lo(w[k]);
                v[2 * k + 1] = bf_hi(w[k]);
            }
        }
        uint4 h = make_uint4(pack2bf(acc[0] + v[0], acc[1] + v[1]), pack2bf(acc[2] + v[2], acc[3] + v[3]),
                             pack2bf(acc[4] + v[4], acc[5] + v[5]), pack2bf(acc[6] + v[6], acc[7] + v[7]));
        if (R) {
            const uint4 x = *reinterpret_cast<const uint4*>(R + (size_t)row * ntot + 8 * c);
            h.x = pack2bf(bf_lo(x.x) + bf_lo(h.x), bf_hi(x.x) + bf_hi(h.x));
            h.y = pack2bf(bf_lo(x.y) + bf_lo(h.y), bf_hi(x.y) + bf_hi(h.y));
            h.z = pack2bf(bf_lo(x.z) + bf_lo(h.z), bf_hi(x.z) + bf_hi(h.z));
            h.w = pack2bf(bf_lo(x.w) + bf_lo(h.w), bf_hi(x.w) + bf_hi(h.w));
        }
        hv[i] = h;
        *reinterpret_cast<uint4*>(C + 8 * c) = h;
        const uint32_t e[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float lo = bf_lo(e[k]), hi = bf_hi(e[k]);
            ss = __builtin_fmaf(lo, lo, ss);
            ss = __builtin_fmaf(hi, hi, ss);
        }
    }
    if (!g.norm_out) return;
    ss = row_wave_sum(ss);
    if ((tid & 63) == 0) wsum[tid >> 6] = ss;
    __syncthreads();
    const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    const float inv = 1.0f / sqrtf(tot / (float)ntot + g.norm_eps);
    const uint16_t* gs = static_cast<const uint16_t*>(g.norm_g);
    uint16_t* n = static_cast<uint16_t*>(g.norm_out) + (size_t)row * ntot;
#pragma unroll
    for (int i = 0; i < kRowsMaxChunks; ++i) {
        const int c = tid + 256 * i;
        if (c >= nch) continue;
        const uint4 v = hv[i], sc = *reinterpret_cast<const uint4*>(gs + 8 * c);
        uint4 o;
        o.x = pack2bf(bf_lo(v.x) * inv * bf_lo(sc.x), bf_hi(v.x) * inv * bf_hi(sc.x));
        o.y = pack2bf(bf_lo(v.y) * inv * bf_lo(sc.y), bf_hi(v.y) * inv * bf_hi(sc.y));
        o.z = pack2bf(bf_lo(v.z) * inv * bf_lo(sc.z), bf_hi(v.z) * inv * bf_hi(sc.z));
        o.w = pack2bf(bf_lo(v.w) * inv * bf_lo(sc.w), bf_hi(v.w) * inv * bf_hi(sc.w));
        *reinterpret_cast<uint4*>(n + 8 * c) = o;
    }
}

// Mid-size row counts (decode of a few hundred sequences): 128 x 128 output tiles, four waves
// of 64 x 64 (2 x 2 tiles of v_mfma_f32_32x32x16_bf16).  At such M the 256 x 256 tiles leave
// 10..60 tiles per projection, and filling the chip then takes K splits whose fp32 partial sums
// outweigh the weights several times over (M Ntot 4 bytes per split against N K 2 for the
// weights); quarter-size tiles need a quarter of the splits or none.  K advances through a ring
// of four LDS stages (64 k per stage, the swizzled 128-byte rows of the large kernel), three
// k-steps of copies in flight ahead of the MFMAs: a split of K may be only a few k-steps long,
// so the ring is filled once and streamed without a refill bubble per step.
constexpr int kMidM = 128, kMidN = 128;
constexpr int kMidStages = 4;
constexpr int kMidMaxRows = 1024;   // 64 < M <= this, one GEMM (no batch), bf16 output

// One operand's copies of k-step kt into an LDS stage of a 128-row tile: 16 copies of 1 KB,
// four per wave (copy 4 w + j fills LDS chunks 64 (4 w + j) .. + 63).  Rows past `rows` repeat
// the last row (results never stored).
__device__ __forceinline__ void copy_mid(const u32x4& rs, uint16_t* lds, int wv, int lane, int K,
                                         int rows, int kt, int row_off = 0) {
    int off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int p = (4 * wv + j) * 64 + lane;
        const int r = p / kChunks;
        const int c = chunk_pos(r, p % kChunks);
        off[j] = (min(r, rows - 1) - row_off) * K * 2 + kt * kRowBytes + 16 * c;
    }
    copy4(rs, lds_address(lds + 4 * wv * 512), off);
}

// K splits of the mid kernel: enough workgroups to cover the chip once (one workgroup per CU:
// the ring takes 128 KB of LDS), at least two k-steps per split.  Split s takes k-steps
// [s KT / S, (s + 1) KT / S).
int mid_ksplit(int M, int Ntot, int K) {
    const long long tiles = (long long)((M + kMidM - 1) / kMidM) * (Ntot / kMidN);
    if (tiles <= 0) return 1;
    long long s = 256 / tiles;
    s = std::min<long long>(s, K / kBK / 2);
    return (int)std::max<long long>(s, 1);
}

// kGated (no K split; two segments of equal width, gate and up): a tile takes 64 features of
// both, the gate rows in tile columns 0..63 and the up rows of the same features in 64..127, so
// waves (wm, 0) and (wm, 1) hold gate and up of the same outputs in the same registers; the up
// half hands its rounded values over through LDS and the gate half writes
// gelu_tanh(gate) * up, rounded as the separate gating step rounds it.
// the mid kernel takes the gating (in its epilogue, or in the split reduction) above the row
// kernel's rows
__host__ __device__ inline bool proj_gemm_mid_gated(int M) { return M > kRowsMax && M <= kMidMaxRows; }

template <bool kSplitK, bool kGated = false>
__global__ void __launch_bounds__(kThreads, 1) proj_gemm_mid_kernel(ProjGemmArgs g) {
    static_assert(!(kSplitK && kGated), "the gating of split sums runs in the reduction");
    __shared__ __attribute__((aligned(16))) uint16_t sa[kMidStages][kMidM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t sb[kMidStages][kMidN * kBK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;
    const int ntot = g.Nw[0] + g.Nw[1] + g.Nw[2];
    const int ntm = (g.M + kMidM - 1) / kMidM, ntn = kGated ? g.Nw[0] / 64 : ntot / kMidN;
    const int S = kSplitK ? g.ksplit : 1;
    // workgroups go to the 8 XCDs round-robin: each XCD gets a contiguous range of the order
    // (M tiles fastest, then N tiles, then splits), so the tiles of one weight block share an L2
    const int total = ntm * ntn * S, bid = (int)blockIdx.x;
    const int L = (total & 7) == 0 ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
    const int m0 = __builtin_amdgcn_readfirstlane(L % ntm) * kMidM;
    const int n0 = __builtin_amdgcn_readfirstlane((L / ntm) % ntn) * (kGated ? 64 : kMidN);
    const int ks = kSplitK ? __builtin_amdgcn_readfirstlane(L / (ntm * ntn)) : 0;
    const int seg = n0 < g.Nw[0] ? 0 : (n0 < g.Nw[0] + g.Nw[1] ? 1 : 2);
    const int nl0 = n0 - (seg > 0 ? g.Nw[0] : 0) - (seg > 1 ? g.Nw[1] : 0);
    const int K = g.K, KT = K / kBK;
    const int kt0 = ks * KT / S, nk = (ks + 1) * KT / S - kt0;
    const int rows = min(g.M - m0, kMidM);
    const uint16_t* A = static_cast<const uint16_t*>(g.A) + (size_t)m0 * K + (size_t)kt0 * kBK;
    // gated: waves 2 and 3 copy tile rows 64..127, the up rows of the same features
    const int wseg = kGated && wv >= 2 ? 1 : seg, wrow_off = kGated && wv >= 2 ? 64 : 0;
    const uint16_t* W = static_cast<const uint16_t*>(g.W[wseg]) + (size_t)nl0 * K + (size_t)kt0 * kBK;
    // (the ranges run kt0 k-steps past the last row's share; no access reaches that far)
    const u32x4 ra = rsrc_words(A, (uint32_t)(rows * K * 2));
    const u32x4 rb = rsrc_words(W, (uint32_t)(kMidN * K * 2));

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    guard_vmem_sgprs(ra, rb);
#pragma unroll
    for (int q = 0; q < kMidStages - 1; ++q)
        if (q < nk) {
            copy_mid(ra, sa[q], wv, lane, K, rows, q);
            copy_mid(rb, sb[q], wv, lane, K, kMidN, q, wrow_off);
        }
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's copies of k-step kt have landed once at most those of the later k-steps
        // already issued (eight loads each) are outstanding; the barrier then publishes the
        // stage, and every wave is past its reads of the stage refilled next (k-step kt - 1)
        const int ahead = min(kMidStages - 2, nk - 1 - kt);
        static_assert(kMidStages == 4, "the waits below cover two later k-steps");
        if (ahead >= 2) wait_vmcnt<16>();
        else if (ahead == 1) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        lds_sync();
        if (kt + kMidStages - 1 < nk) {
            const int st = (kt + kMidStages - 1) % kMidStages;
            copy_mid(ra, sa[st], wv, lane, K, rows, kt + kMidStages - 1);
            copy_mid(rb, sb[st], wv, lane, K, kMidN, kt + kMidStages - 1, wrow_off);
        }
        const uint16_t* ca = sa[kt % kMidStages];
        const uint16_t* cb = sb[kt % kMidStages];
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = frag(ca, 64 * wm + 32 * i, lane, s);
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = frag(cb, 64 * wn + 32 * j, lane, s);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
    }

    // acc[i][j] is the transposed 32 x 32 tile: lane l holds output row 32 i + l % 32 and, in
    // registers 4 q .. 4 q + 3, output columns 32 j + 8 q + 4 (l / 32) + 0..3 (wave offsets added)
    const int ncol = 64 * wn + 4 * (lane >> 5);
    const int mrow = 64 * wm + (lane & 31);
    if constexpr (kGated) {
        // gate (wn = 0) and up (wn = 1) of features n0 + 32 j + 8 q + 4 (l / 32) + 0..3, rounded
        // with their biases; up through LDS (stage memory, free once every wave is past its
        // last MFMA operands)
        const uint16_t* bias = static_cast<const uint16_t*>(g.b[wn]);
        u32x2 gv[2][2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = n0 + 4 * (lane >> 5) + 32 * j + 8 * q;
                const uint2 bw = bias ? *reinterpret_cast<const uint2*>(bias + f) : make_uint2(0u, 0u);
                const float bv[4] = {bf_lo(bw.x), bf_hi(bw.x), bf_lo(bw.y), bf_hi(bw.y)};
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const f32x16& t = acc[i][j];
                    gv[i][j][q] = u32x2{pack2bf(t[4 * q] + bv[0], t[4 * q + 1] + bv[1]),
                                        pack2bf(t[4 * q + 2] + bv[2], t[4 * q + 3] + bv[3])};
                }
            }
        u32x2* const xb = reinterpret_cast<u32x2*>(&sa[0][0]) + wm * (2 * 2 * 4 * 64);
        __syncthreads();
        if (wn == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) xb[((i * 2 + j) * 4 + q) * 64 + lane] = gv[i][j][q];
        }
        __syncthreads();
        if (wn == 1) return;
        const int ldc = g.Nw[0];
        uint16_t* C = static_cast<uint16_t*>(g.C[0]) + (size_t)m0 * ldc + n0;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc_n(C, (uint32_t)(rows * ldc * 2));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 gt = gv[i][j][q], up = xb[((i * 2 + j) * 4 + q) * 64 + lane];
                    const u32x2 v = {pack2bf(gelu_fast(bf_lo(gt[0])) * bf_lo(up[0]), gelu_fast(bf_hi(gt[0])) * bf_hi(up[0])),
                                     pack2bf(gelu_fast(bf_lo(gt[1])) * bf_lo(up[1]), gelu_fast(bf_hi(gt[1])) * bf_hi(up[1]))};
                    const int off = ((mrow + 32 * i) * ldc + 4 * (lane >> 5) + 32 * j + 8 * q) * 2;
                    __builtin_amdgcn_raw_buffer_store_b64(v, rc, off, 0, 0);
                }
        return;
    }
    if constexpr (kSplitK) {
        float* P = g.part + ((size_t)ks * g.M + m0) * ntot + n0;
        const __amdgpu_buffer_rsrc_t rp = make_rsrc_n(P, (uint32_t)(rows * ntot * 4));
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const f32x16& t = acc[i][j];
                    const f32x4 v = {t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
                    const int off = ((mrow + 32 * i) * ntot + ncol + 32 * j + 8 * q) * 4;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp, off,
                                                           0, 0);
                }
        return;
    }
    const uint16_t* bias = static_cast<const uint16_t*>(g.b[seg]);
    const int ldc = g.Nw[seg];
    uint16_t* C = static_cast<uint16_t*>(g.C[seg]) + (size_t)m0 * ldc + nl0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc_n(C, (uint32_t)(rows * ldc * 2));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = ncol + 32 * j + 8 * q;
            const uint2 bw = bias ? *reinterpret_cast<const uint2*>(bias + nl0 + n) : make_uint2(0u, 0u);
            const float bv[4] = {bf_lo(bw.x), bf_hi(bw.x), bf_lo(bw.y), bf_hi(bw.y)};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x16& t = acc[i][j];
                const u32x2 v = {pack2bf(t[4 * q] + bv[0], t[4 * q + 1] + bv[1]),
                                 pack2bf(t[4 * q + 2] + bv[2], t[4 * q + 3] + bv[3])};
                const int off = ((mrow + 32 * i) * ldc + n) * 2;
                __builtin_amdgcn_raw_buffer_store_b64(v, rc, off, 0, 0);
            }
        }
    }
}

// Few rows, up to 64, where the row kernel below does not apply and the caller gives no
// partial-sum space (a Linear without a workspace).  One workgroup per 16 output features: the weight rows are the A operand of
// v_mfma_f32_16x16x32_bf16 (16 features x 32 k, each lane 16 bytes of one row) and up to 64
// input rows the B operand in blocks of 16 columns, so each weight byte is read once and no
// MFMA work is spent on rows that do not exist.  The eight waves take an eighth of K each, with
// eight weight loads in flight per wave (a few waves per CU must keep enough bytes in flight to
// stream the weights); their tiles are added in wave order through LDS.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kSkinnyWaves = 8;
template <int NB>   // blocks of 16 input rows: M <= 16 NB
__global__ void __launch_bounds__(64 * kSkinnyWaves) skinny_gemm_kernel(ProjGemmArgs g) {
    __shared__ f32x4 red[kSkinnyWaves][NB][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * 16;
    const int seg = n0 < g.Nw[0] ? 0 : (n0 < g.Nw[0] + g.Nw[1] ? 1 : 2);
    const int nl0 = n0 - (seg > 0 ? g.Nw[0] : 0) - (seg > 1 ? g.Nw[1] : 0);
    const int K = g.K, kq = K / kSkinnyWaves, g16 = lane >> 4;   // kq % 32 == 0
    const uint16_t* W = static_cast<const uint16_t*>(g.W[seg]) + (size_t)(nl0 + (lane & 15)) * K;
    const uint16_t* X = static_cast<const uint16_t*>(g.A);
    int xr[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xr[b] = min(16 * b + (lane & 15), g.M - 1);
    f32x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int kb = wv * kq + 8 * g16, ke = (wv + 1) * kq;
#pragma unroll 8
    for (int k = kb; k < ke; k += 32) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(W + k);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            // rows past M repeat the last row; their columns are never stored
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(X + (size_t)xr[b] * K + k);
            acc[b] = mfma16(a, x, acc[b]);
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) red[wv][b][lane] = acc[b];
    __syncthreads();
    if (tid >= NB * 64) return;
    // lane l of block b: input row 16 b + l % 16, features 4 (l / 16) .. + 3
    const int b = tid >> 6, l = tid & 63, m = 16 * b + (l & 15);
    if (m >= g.M) return;
    f32x4 t = red[0][b][l];
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w) t += red[w][b][l];
    const int n = nl0 + 4 * (l >> 4);
    const uint16_t* bias = static_cast<const uint16_t*>(g.b[seg]);
    float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (bias) {
        const uint2 bw = *reinterpret_cast<const uint2*>(bias + n);
        bv[0] = bf_lo(bw.x); bv[1] = bf_hi(bw.x); bv[2] = bf_lo(bw.y); bv[3] = bf_hi(bw.y);
    }
    uint16_t* C = static_cast<uint16_t*>(g.C[seg]) + (size_t)m * g.Nw[seg] + n;
    *reinterpret_cast<uint2*>(C) = make_uint2(pack2bf(t[0] + bv[0], t[1] + bv[1]),
                                              pack2bf(t[2] + bv[2], t[3] + bv[3]));
}

// One to four rows with K % 512 == 0 (decode of one to four sequences).  One wave per output
// feature: lane l takes the 16-byte pieces k = 512 c + 8 l of the feature's weight row, so every
// load instruction reads 1 KB of one row contiguously (the MFMA kernel above reads 64 bytes of
// each of 16 rows per instruction and streams the weights about 1.5x slower at these sizes).
// Pairs of bf16 products accumulate in fp32 with v_dot2_f32_bf16; a butterfly over the wave
// then adds the 64 lanes' sums, the same order for every feature and call.
//
// Two epilogues serve the layer's MLP (page "Gemma 詳解：RecurrentGemma 架構", the MLP block of
// the residual layers) without extra launches, with the roundings of the separate steps:
//   kGated  the wave takes feature n of both segments (gate and up rows) and writes
//           gelu_tanh(gate) * up, each rounded to bf16 first, as the gating step would;
//   R       the final residual addition: C = R + the bf16 output, rounded again.
typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16v2, a),
                                           __builtin_bit_cast(bf16v2, b), c, false);
}
__device__ __forceinline__ void dot8(const uint4& w, const uint4& x, float& acc) {
    acc = dot2(w.x, x.x, acc);
    acc = dot2(w.y, x.y, acc);
    acc = dot2(w.z, x.z, acc);
    acc = dot2(w.w, x.w, acc);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

constexpr int kRowsWaves = 4;      // features (waves) per workgroup
// kNorm: the input rows are normalised on the way in (in_norm_g).  Each wave first forms every
// row's sum of squares over the same 8-element chunks per lane (chunk lane + 64 i), in the same
// order and with the same butterfly as the norm kernel, so each normalised input is bitwise
// what that kernel would have written; the row is 2 * K bytes, read again from the cache by the
// main loop.
template <int NB, bool kGated, bool kNorm>   // input rows held per lane: M <= NB
__global__ void __launch_bounds__(64 * kRowsWaves) gemv_rows_kernel(ProjGemmArgs g) {
    constexpr int NS = kGated ? 2 : 1;   // weight rows per wave
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * kRowsWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = kGated ? 0 : (n < g.Nw[0] ? 0 : (n < g.Nw[0] + g.Nw[1] ? 1 : 2));
    const int nl = n - (seg > 0 ? g.Nw[0] : 0) - (seg > 1 ? g.Nw[1] : 0);
    const int K = g.K;
    const uint16_t* w[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j)
        w[j] = static_cast<const uint16_t*>(g.W[seg + j]) + (size_t)nl * K + 8 * lane;
    const uint16_t* x = static_cast<const uint16_t*>(g.A) + 8 * lane;
    size_t xo[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xo[b] = (size_t)min(b, g.M - 1) * K;   // rows past M repeat
    float inv[NB];
    const uint16_t* gs = static_cast<const uint16_t*>(g.in_norm_g) + 8 * lane;
    if constexpr (kNorm) {
        float ss[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) ss[b] = 0.0f;
#pragma unroll 4
        for (int k = 0; k < K; k += 512) {
            uint4 v[NB];   // every row's chunk in flight together
#pragma unroll
            for (int b = 0; b < NB; ++b) v[b] = *reinterpret_cast<const uint4*>(x + xo[b] + k);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint32_t e[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = bf_lo(e[q]), hi = bf_hi(e[q]);
                    ss[b] = __builtin_fmaf(lo, lo, ss[b]);
                    ss[b] = __builtin_fmaf(hi, hi, ss[b]);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) inv[b] = 1.0f / sqrtf(wave_sum(ss[b]) / (float)K + g.in_norm_eps);
    }
    float acc[NS][NB];
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[j][b] = 0.0f;
#pragma unroll 4
    for (int k = 0; k < K; k += 512) {
        uint4 wv[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) wv[j] = *reinterpret_cast<const uint4*>(w[j] + k);
        uint4 sv;
        if constexpr (kNorm) sv = *reinterpret_cast<const uint4*>(gs + k);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint4 xv = *reinterpret_cast<const uint4*>(x + xo[b] + k);
            if constexpr (kNorm) {
                const float t = inv[b];
                xv.x = pack2bf(bf_lo(xv.x) * t * bf_lo(sv.x), bf_hi(xv.x) * t * bf_hi(sv.x));
                xv.y = pack2bf(bf_lo(xv.y) * t * bf_lo(sv.y), bf_hi(xv.y) * t * bf_hi(sv.y));
                xv.z = pack2bf(bf_lo(xv.z) * t * bf_lo(sv.z), bf_hi(xv.z) * t * bf_hi(sv.z));
                xv.w = pack2bf(bf_lo(xv.w) * t * bf_lo(sv.w), bf_hi(xv.w) * t * bf_hi(sv.w));
            }
#pragma unroll
            for (int j = 0; j < NS; ++j) dot8(wv[j], xv, acc[j][b]);
        }
    }
    float bv[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const uint16_t* bias = static_cast<const uint16_t*>(g.b[seg + j]);
        bv[j] = bias ? bf2f(bias[nl]) : 0.0f;
    }
    const int ldc = kGated ? g.Nw[0] : g.Nw[seg];
    uint16_t* C = static_cast<uint16_t*>(g.C[seg]) + nl;
    const uint16_t* R = static_cast<const uint16_t*>(g.R);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float v = bf2f(f2bf(wave_sum(acc[0][b]) + bv[0]));
        if (kGated) v = gelu_fast(v) * bf2f(f2bf(wave_sum(acc[1][b]) + bv[1]));
        else if (R) v += bf2f(R[(size_t)min(b, g.M - 1) * ldc + nl]);
        if (lane == b && b < g.M) C[(size_t)b * ldc] = f2bf(v);
    }
}

// K splits for a shape: enough blocks to cover the chip (about 240) when the tiles alone do
// not, each split a multiple of 128 of K.
int choose_ksplit(int M, int Ntot, int K, int batch = 1) {
    const long long tiles = (long long)((M + kBM - 1) / kBM) * (Ntot / kBN) * (batch > 1 ? batch : 1);
    if (tiles <= 0 || tiles >= 240) return 1;
    const int want = (int)((240 + tiles - 1) / tiles), units = K / 128;
    int best = 1;
    for (int s = 1; s <= units && s <= want; ++s)
        if (units % s == 0) best = s;
    return best;
}

}  // namespace

bool proj_gemm_rows(int M, int K) { return M >= 1 && M <= kRowsMax && K % 512 == 0; }

bool proj_gemm_gated_ok(int M, int K) { return proj_gemm_rows(M, K) || M > kRowsMax; }

size_t proj_gemm_part_bytes(int M, int Ntot, int K) {
    if (proj_gemm_rows(M, K)) return 0;
    const int s = M <= kMidMaxRows ? mid_ksplit(M, Ntot, K) : choose_ksplit(M, Ntot, K);
    return s > 1 ? (size_t)s * M * Ntot * sizeof(float) : 0;
}

bool proj_gemm_rows_epilogue_ok(int M) { return M > kRowsMax; }

size_t proj_gemm_part_bytes_rows_epilogue(int M, int Ntot, int K) {
    if (!proj_gemm_rows_epilogue_ok(M)) return 0;
    const int s = M <= kMidMaxRows ? mid_ksplit(M, Ntot, K) : choose_ksplit(M, Ntot, K);
    return (size_t)std::max(s, 1) * M * Ntot * sizeof(float);
}

size_t proj_gemm_part_bytes_batched(int batch, int M, int Ntot, int K) {
    if (batch <= 1) return proj_gemm_part_bytes(M, Ntot, K);
    const int s = choose_ksplit(M, Ntot, K, batch);
    return s > 1 ? (size_t)batch * s * M * Ntot * sizeof(float) : 0;
}

hipError_t launch_proj_gemm(const ProjGemmArgs& a_in, hipStream_t s) {
    ProjGemmArgs a = a_in;
    a.ntm = (a.M + kBM - 1) / kBM;
    a.ntn = (a.Nw[0] + a.Nw[1] + a.Nw[2]) / kBN;
    const long long tiles = (long long)a.ntm * a.ntn;
    if (tiles <= 0) return hipSuccess;
    a.ksplit = 1;
    const int nb = a.batch > 1 ? a.batch : 1;
    if (nb > 1) {
        // a batch runs on the tile kernel only
        if (a.gated || a.R || a.rows_epilogue || a.in_norm_g) return hipErrorInvalidValue;
        if (a.part) {
            const int ks = choose_ksplit(a.M, a.ntn * kBN, a.K, nb);
            if (ks > 1 && (size_t)nb * ks * a.M * a.ntn * kBN * sizeof(float) <= a.part_bytes) a.ksplit = ks;
        }
        if (a.c_f32 && a.ksplit == 1) return hipErrorInvalidValue;
        if (a.ksplit > 1)
            hipLaunchKernelGGL(proj_gemm_kernel<true>, dim3((unsigned)(nb * tiles * a.ksplit)),
                               dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL(proj_gemm_kernel<false>, dim3((unsigned)(nb * tiles)), dim3(kThreads), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.ksplit == 1) return e;
        const size_t n = (size_t)nb * a.M * a.ntn * kBN / 8;
        hipLaunchKernelGGL(proj_splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           s, a);
        return hipGetLastError();
    }
    if (a.rows_epilogue) {
        // partials (even unsplit) on a tile kernel, then one wave per row adds them with the
        // bias, R and the norm
        const int ntot = a.ntn * kBN;
        if (a.nseg != 1 || a.gated || a.c_f32 || a.in_norm_g || !proj_gemm_rows_epilogue_ok(a.M) || !a.part ||
            ntot > 8 * 256 * kRowsMaxChunks || (a.norm_out && !a.norm_g))
            return hipErrorInvalidValue;
        const bool mid = a.M <= kMidMaxRows;
        int ks = std::max(mid ? mid_ksplit(a.M, ntot, a.K) : choose_ksplit(a.M, ntot, a.K), 1);
        while (ks > 1 && (size_t)ks * a.M * ntot * sizeof(float) > a.part_bytes) --ks;
        if ((size_t)ks * a.M * ntot * sizeof(float) > a.part_bytes) return hipErrorInvalidValue;
        a.ksplit = ks;
        if (mid)
            hipLaunchKernelGGL(proj_gemm_mid_kernel<true>,
                               dim3((unsigned)(((a.M + kMidM - 1) / kMidM) * (ntot / kMidN) * ks)),
                               dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL(proj_gemm_kernel<true>, dim3((unsigned)(tiles * ks)), dim3(kThreads), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(proj_splitk_rows_kernel, dim3((unsigned)a.M), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const bool rows = !a.c_f32 && proj_gemm_rows(a.M, a.K);
    if (a.gated && !((rows || (!a.c_f32 && a.M > kRowsMax)) && a.nseg == 2 && a.Nw[0] == a.Nw[1]))
        return hipErrorInvalidValue;
    if (a.R && !(rows && a.nseg == 1)) return hipErrorInvalidValue;
    if (a.in_norm_g && !rows) return hipErrorInvalidValue;
    if (rows) {
        const unsigned blocks = (unsigned)((a.gated ? a.Nw[0] : a.ntn * kBN) / kRowsWaves);
        const dim3 grid(blocks), blk(64 * kRowsWaves);
        const int nb = a.M == 1 ? 1 : (a.M == 2 ? 2 : 4);
#define RG_ROWS(G, NORM)                                                                      \
        switch (nb) {                                                                         \
            case 1: hipLaunchKernelGGL((gemv_rows_kernel<1, G, NORM>), grid, blk, 0, s, a); break; \
            case 2: hipLaunchKernelGGL((gemv_rows_kernel<2, G, NORM>), grid, blk, 0, s, a); break; \
            default: hipLaunchKernelGGL((gemv_rows_kernel<4, G, NORM>), grid, blk, 0, s, a);  \
        }
        if (a.gated) {
            if (a.in_norm_g) { RG_ROWS(true, true) } else { RG_ROWS(true, false) }
        } else {
            if (a.in_norm_g) { RG_ROWS(false, true) } else { RG_ROWS(false, false) }
        }
#undef RG_ROWS
        return hipGetLastError();
    }
    // the skinny kernel's waves each take whole 32-wide steps of K: K % (32 * waves) == 0.  With
    // partial-sum space the mid-size tiles and their K splits serve these rows instead: a 128-row
    // tile reads each weight byte once too, and the splits cover the chip (at 64 rows the
    // 26-layer decode step took 2.84 ms that way against 4.76 ms with this kernel).
    if (!a.c_f32 && !a.part && !a.gated && a.M <= kSkinnyRows && a.K % (32 * kSkinnyWaves) == 0) {
        const unsigned blocks = (unsigned)(a.ntn * kBN / 16);
        switch ((a.M + 15) / 16) {
            case 1: hipLaunchKernelGGL(skinny_gemm_kernel<1>, dim3(blocks), dim3(512), 0, s, a); break;
            case 2: hipLaunchKernelGGL(skinny_gemm_kernel<2>, dim3(blocks), dim3(512), 0, s, a); break;
            case 3: hipLaunchKernelGGL(skinny_gemm_kernel<3>, dim3(blocks), dim3(512), 0, s, a); break;
            default: hipLaunchKernelGGL(skinny_gemm_kernel<4>, dim3(blocks), dim3(512), 0, s, a);
        }
        return hipGetLastError();
    }
    if (!a.c_f32 && a.M <= kMidMaxRows) {
        const int ntot = a.ntn * kBN;
        if (a.part) {
            const int ks = mid_ksplit(a.M, ntot, a.K);
            if (ks > 1 && (size_t)ks * a.M * ntot * sizeof(float) <= a.part_bytes) a.ksplit = ks;
        }
        const unsigned ntm = (unsigned)((a.M + kMidM - 1) / kMidM);
        const unsigned blocks = ntm * (unsigned)(ntot / kMidN) * (unsigned)a.ksplit;
        if (a.ksplit > 1)
            hipLaunchKernelGGL((proj_gemm_mid_kernel<true, false>), dim3(blocks), dim3(kThreads), 0, s, a);
        else if (a.gated)
            hipLaunchKernelGGL((proj_gemm_mid_kernel<false, true>), dim3(ntm * (unsigned)(a.Nw[0] / 64)),
                               dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((proj_gemm_mid_kernel<false, false>), dim3(blocks), dim3(kThreads), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.ksplit == 1) return e;
        const size_t n = (size_t)a.M * (a.gated ? a.Nw[0] : ntot) / 8;
        hipLaunchKernelGGL(proj_splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, s, a);
        return hipGetLastError();
    }
    if (a.part) {
        const int ks = choose_ksplit(a.M, a.ntn * kBN, a.K);
        if (ks > 1 && (size_t)ks * a.M * a.ntn * kBN * sizeof(float) <= a.part_bytes) a.ksplit = ks;
    }
    if (a.c_f32 && a.ksplit == 1) return hipErrorInvalidValue;   // fp32 output needs the split path
    if (a.ksplit > 1)
        hipLaunchKernelGGL(proj_gemm_kernel<true>, dim3((unsigned)(tiles * a.ksplit)),
                           dim3(kThreads), 0, s, a);
    else if (a.gated)
        hipLaunchKernelGGL((proj_gemm_kernel<false, true>), dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((proj_gemm_kernel<false, false>), dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.ksplit == 1) return e;
    const size_t n = (size_t)a.M * (a.gated ? a.Nw[0] : a.ntn * kBN) / 8;
    hipLaunchKernelGGL(proj_splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace rglru
