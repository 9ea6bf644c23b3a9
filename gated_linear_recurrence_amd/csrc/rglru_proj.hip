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
// weight and write x, the others read linear_y's weight and write y.
//
// Workgroup tile 256 x 256, four waves of 128 x 128 (4 x 4 tiles of v_mfma_f32_32x32x16_bf16,
// 256 fp32 accumulators per lane).  K advances in steps of 32 through a ring of four LDS stages
// filled by buffer loads with the LDS bit (16 bytes per lane, straight into LDS), three steps
// ahead of the MFMAs.  Each stage is its own LDS array: the compiler can then tell a stage being
// read from the copies in flight into the others, and does not wait for those copies.
#include "rglru_device.h"
#include "rglru_internal.h"

namespace rglru {
namespace {

typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

constexpr int kBM = 256;                    // tile rows (M)
constexpr int kBN = 256;                    // tile columns (N)
constexpr int kBK = 32;                     // K per stage
constexpr int kThreads = 256;               // 4 waves, 2 x 2 over the tile
constexpr int kChunks = kBK / 8;            // 16-byte chunks per tile row
constexpr int kRowBytes = kBK * 2;
constexpr int kTileBytes = kBM * kRowBytes;             // one operand, one stage: 16 KB
constexpr int kCopiesPerWave = kTileBytes / 1024 / 4;   // 1 KB copies per wave, operand, stage
constexpr int kGroupM = 8;                  // tile rows per group of the tile order
static_assert(kBM == kBN, "both operands share the copy and fragment helpers");
static_assert(kChunks == 4, "the chunk swizzle below is written for 64-byte rows");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Position of 16-byte chunk c of tile row r inside the row.  A ds_read_b128 serves 8 lanes
// (8 consecutive rows, one chunk index) per pass; with 64-byte rows, rows r and r + 1 share a
// 128-byte bank line, so chunk c of row r goes to c ^ ((r / 2) % 4): the 8 rows then cover all
// 8 16-byte bank groups.
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ ((r >> 1) & 3); }

// Copy k-step kt of one operand's 256 tile rows into an LDS stage.  Tile row r is global row
// min(r, rows - 1) relative to the resource base: rows past a ragged M repeat the last row and
// their results are never stored.  Each copy moves 1 KB: lane l of copy q fills LDS chunk
// 64 q + l, so the global side picks the chunk that belongs there.
__device__ __forceinline__ void copy_stage(__amdgpu_buffer_rsrc_t rs, uint16_t* lds, int wv,
                                           int lane, int K, int rows, int kt) {
#pragma unroll
    for (int j = 0; j < kCopiesPerWave; ++j) {
        const int q = wv * kCopiesPerWave + j;
        const int p = q * 64 + lane;
        const int r = p / kChunks;
        const int c = chunk_pos(r, p % kChunks);   // the swizzle is its own inverse
        const int off = min(r, rows - 1) * K * 2 + kt * kRowBytes + 16 * c;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds + q * 512, 16, off, 0, 0, 0);
    }
}

// A or B fragment of the 32-row tile starting at row r0, K sub-step s (16 k): lane l supplies
// row r0 + l % 32 and k = 16 s + 8 (l / 32) .. + 7.
__device__ __forceinline__ bf16x8 frag(const uint16_t* lds, int r0, int lane, int s) {
    const int r = r0 + (lane & 31);
    const int c = 2 * s + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(lds + r * kBK + 8 * chunk_pos(r, c));
}

__device__ __forceinline__ void mma_stage(const uint16_t* sa, const uint16_t* sb,
                                          f32x16 (&acc)[4][4], int wm, int wn, int lane) {
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
        bf16x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = frag(sa, 128 * wm + 32 * i, lane, s);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = frag(sb, 128 * wn + 32 * j, lane, s);
        // weight rows as the MFMA's A operand: the result tile is C^T, so each lane ends up
        // with 4 consecutive output columns per register group (8-byte stores)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
}

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Barrier over LDS accesses (each wave has waited for its own copies before it arrives).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

__global__ void __launch_bounds__(kThreads, 1) proj_gemm_kernel(ProjGemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint16_t a0[kBM * kBK], a1[kBM * kBK], a2[kBM * kBK],
        a3[kBM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t b0[kBN * kBK], b1[kBN * kBK], b2[kBN * kBK],
        b3[kBN * kBK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (the copies' LDS base)
    const int wm = wv >> 1, wn = wv & 1;
    int tm, tn;
    tile_of(blockIdx.x, g.ntm, g.ntn, tm, tn);
    // the divisions above run on the vector unit; the tile is uniform, and the buffer resources
    // built from it must sit in scalar registers
    const int m0 = __builtin_amdgcn_readfirstlane(tm) * kBM;
    const int n0 = __builtin_amdgcn_readfirstlane(tn) * kBN;
    const bool second = n0 >= g.N0;               // the y half of the branch projections
    const int nl0 = second ? n0 - g.N0 : n0;
    const int K = g.K;
    const int rows = min(g.M - m0, kBM);
    const uint16_t* A = static_cast<const uint16_t*>(g.A) + (size_t)m0 * K;
    const uint16_t* W = static_cast<const uint16_t*>(second ? g.W1 : g.W0) + (size_t)nl0 * K;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc_n(A, (uint32_t)(rows * K * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc_n(W, (uint32_t)(kBN * K * 2));
    const int KT = K / kBK;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // three k-steps in flight before the first MFMA
    copy_stage(ra, a0, wv, lane, K, rows, 0);
    copy_stage(rb, b0, wv, lane, K, kBN, 0);
    if (KT > 1) {
        copy_stage(ra, a1, wv, lane, K, rows, 1);
        copy_stage(rb, b1, wv, lane, K, kBN, 1);
    }
    if (KT > 2) {
        copy_stage(ra, a2, wv, lane, K, rows, 2);
        copy_stage(rb, b2, wv, lane, K, kBN, 2);
    }

    // one k-step: wait for this wave's copies of stage kt (those of the next two steps may stay
    // in flight), meet the other waves (their copies have landed, and nobody still reads the
    // stage about to be refilled), refill it three steps ahead, then run the MFMAs
    auto step = [&](int kt, const uint16_t* ca, const uint16_t* cb, uint16_t* na, uint16_t* nb) {
        constexpr int kPerStep = 2 * kCopiesPerWave;
        const int ahead = KT - 1 - kt;
        if (ahead >= 2) wait_vmcnt<2 * kPerStep>();
        else if (ahead == 1) wait_vmcnt<kPerStep>();
        else wait_vmcnt<0>();
        lds_sync();
        if (kt + 3 < KT) {
            copy_stage(ra, na, wv, lane, K, rows, kt + 3);
            copy_stage(rb, nb, wv, lane, K, kBN, kt + 3);
        }
        mma_stage(ca, cb, acc, wm, wn, lane);
    };
    // Step 0 runs before the loop, so the loop's first step reads stage 1: with stage 0 read
    // right after the loop header, the compiler's tracking of copies into LDS loses track of
    // which stage each copy targets and waits for all of them there (the just-issued refill
    // included), a full memory round trip every fourth step.  KT % 4 == 0.
    step(0, a0, b0, a3, b3);
    for (int kt = 1; kt < KT; kt += 4) {
        step(kt, a1, b1, a0, b0);
        step(kt + 1, a2, b2, a1, b1);
        step(kt + 2, a3, b3, a2, b2);
        if (kt + 3 < KT) step(kt + 3, a0, b0, a3, b3);
    }

    // bias, round, store.  acc[i][j] is the transposed 32 x 32 tile: lane l holds output row
    // 32 i + l % 32 and, in registers 4 q .. 4 q + 3, output columns 32 j + 8 q + 4 (l / 32) + 0..3.
    // The buffer's range ends at the last valid row, so stores of rows past a ragged M are dropped.
    const uint16_t* bias = static_cast<const uint16_t*>(second ? g.b1 : g.b0);
    const int ldc = g.N0;
    uint16_t* C = static_cast<uint16_t*>(second ? g.C1 : g.C0) + (size_t)m0 * ldc + nl0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc_n(C, (uint32_t)(rows * ldc * 2));
    const int ncol = 128 * wn + 4 * (lane >> 5);
    const int mrow = 128 * wm + (lane & 31);
    uint2 bw[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bw[j][q] = bias ? *reinterpret_cast<const uint2*>(bias + nl0 + ncol + 32 * j + 8 * q)
                            : make_uint2(0u, 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = ncol + 32 * j + 8 * q;
            const float bv[4] = {bf_lo(bw[j][q].x), bf_hi(bw[j][q].x), bf_lo(bw[j][q].y),
                                 bf_hi(bw[j][q].y)};
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

}  // namespace

hipError_t launch_proj_gemm(const ProjGemmArgs& a_in, hipStream_t s) {
    ProjGemmArgs a = a_in;
    a.ntm = (a.M + kBM - 1) / kBM;
    a.ntn = a.n_out * a.N0 / kBN;
    const long long tiles = (long long)a.ntm * a.ntn;
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(proj_gemm_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace rglru
