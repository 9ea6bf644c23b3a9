// Decode step: one token for each of N sequences, updating the carried fp32 state h and the
// three-token conv window in place (the fixed-size state that lets the recurrent block
// generate sequences of any length: page "Gemma 詳解：RecurrentGemma 架構", sections
// "模型寬度與 RNN 寬度" and "區域注意力視窗大小").
//
// Two forms of the bf16 step compute the same expressions:
//  - fused (no workspace): workgroup = (tile of 32 sequences, gate head).  The conv runs over
//    [window, x_t] and shifts the window; u goes to LDS; the gate projections of the 32
//    sequences are one 32-row MFMA tile per wave (32 output channels); then
//    h <- a h + sqrt(1-a^2) i u and out = h * gelu_tanh(y_t).
//  - split (with a workspace): a conv pass writes u and shifts the window, then a gate pass
//    spreads each head's output channels over many workgroups (see the two kernels below).
// fp32 storage uses the fused decomposition with precise gate math.
#include <type_traits>

#include "rglru_device.h"
#include "rglru_internal.h"

namespace rglru {

namespace {

constexpr float kLn2 = 0.6931471805599453f;

// softplus(-L) from hardware exp2/log2 (a few ulp; ~20 instructions instead of the library
// expf/log1pf).  log1p(e) is formed as log(1 + e) * e / ((1 + e) - 1), which cancels the
// rounding of 1 + e (Goldberg's correction), so small e keeps full relative accuracy.
__device__ __forceinline__ float softplus_neg_fast(float lam) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(lam) * kLog2e);  // exp(-|L|) in (0, 1]
    const float w = 1.0f + e;
    const float d = w - 1.0f;
    const float l1p = d == 0.0f ? e : __builtin_amdgcn_logf(w) * kLn2 * (e * __builtin_amdgcn_rcpf(d));
    return fmaxf(-lam, 0.0f) + l1p;
}

// gate_ikc with the hardware reciprocal (1 ulp); rcp(-0) = -inf also maps to -FLT_MAX.
__device__ __forceinline__ float gate_ikc_fast(float sp_neg) {
    return fmaxf(__builtin_amdgcn_rcpf(-8.0f * sp_neg * kLog2e), -3.4028234663852886e38f);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffff, 0x00020000);
}

template <int BS, typename ST>
__global__ void __launch_bounds__(2 * BS) decode_kernel(DecodeArgs a) {
    using S = Store<ST>;
    constexpr bool kBf = S::kBf16;
    constexpr int kChunks = BS / 8;
    constexpr int kGroups = (2 * BS) / kChunks;  // 16 sequence groups of 2
    constexpr int kRow = kBf ? BS + 8 : BS + 4;
    using L = typename std::conditional<kBf, uint16_t, float>::type;
    __shared__ __attribute__((aligned(16))) L u_lds[32 * kRow];

    const int tid = threadIdx.x;
    const int n0 = blockIdx.x * 32;
    const int head = blockIdx.y;
    const int N = a.N;
    const size_t D = (size_t)a.D;
    ST* __restrict__ cs = static_cast<ST*>(a.conv_state);

    // ---- conv over [window, x_t]; shift the window in place ----
    {
        const int cg = tid % kChunks, sg = tid / kChunks;
        const size_t c0 = (size_t)head * BS + cg * 8;
        const ST* cw = static_cast<const ST*>(a.conv_w) + c0 * 4;
        float w[4][8];
        {
            float tmp[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                S::load8(cw + 8 * q, tmp);
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e & 3][2 * q + (e >> 2)] = tmp[e];
            }
        }
        float cb[8];
        if (a.conv_b) S::load8(static_cast<const ST*>(a.conv_b) + c0, cb);
        else {
#pragma unroll
            for (int e = 0; e < 8; ++e) cb[e] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 32 / kGroups; ++k) {
            const int m = sg * (32 / kGroups) + k;
            const int n = n0 + m;
            float u[8];
            if (n < N) {
                float s0[8], s1[8], s2[8], xt[8];
                S::load8(cs + ((size_t)n * 3 + 0) * D + c0, s0);
                S::load8(cs + ((size_t)n * 3 + 1) * D + c0, s1);
                S::load8(cs + ((size_t)n * 3 + 2) * D + c0, s2);
                S::load8(static_cast<const ST*>(a.x) + (size_t)n * a.ld_x + c0, xt);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float acc = __builtin_fmaf(w[0][e], s0[e], cb[e]);
                    acc = __builtin_fmaf(w[1][e], s1[e], acc);
                    acc = __builtin_fmaf(w[2][e], s2[e], acc);
                    u[e] = __builtin_fmaf(w[3][e], xt[e], acc);
                }
                S::store8(cs + ((size_t)n * 3 + 0) * D + c0, s1);
                S::store8(cs + ((size_t)n * 3 + 1) * D + c0, s2);
                S::store8(cs + ((size_t)n * 3 + 2) * D + c0, xt);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) u[e] = 0.0f;
            }
            L* dst = u_lds + m * kRow + cg * 8;
            if constexpr (kBf) {
                *reinterpret_cast<uint4*>(dst) = make_uint4(pack2bf(u[0], u[1]), pack2bf(u[2], u[3]),
                                                            pack2bf(u[4], u[5]), pack2bf(u[6], u[7]));
            } else {
                *reinterpret_cast<float4*>(dst) = make_float4(u[0], u[1], u[2], u[3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(u[4], u[5], u[6], u[7]);
            }
        }
    }
    __syncthreads();

    // ---- gates: one 32x32 tile per gate per wave (rows = sequences) ----
    const int wv = tid >> 6, lane = tid & 63, ln = lane & 31, kh = lane >> 5;
    const int ncol = wv * 32 + ln;
    const size_t ch = (size_t)head * BS + ncol;
    f32x16 accA, accX;
#pragma unroll
    for (int e = 0; e < 16; ++e) { accA[e] = 0.0f; accX[e] = 0.0f; }
    {
        const ST* war = static_cast<const ST*>(a.wa) + ((size_t)head * BS + ncol) * BS;
        const ST* wxr = static_cast<const ST*>(a.wx) + ((size_t)head * BS + ncol) * BS;
        if constexpr (kBf) {
#pragma unroll
            for (int q4 = 0; q4 < BS / 64; ++q4) {
                const int kb = 64 * q4 + 32 * kh;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 bA = *reinterpret_cast<const bf16x8*>(war + kb + 8 * s);
                    const bf16x8 bX = *reinterpret_cast<const bf16x8*>(wxr + kb + 8 * s);
                    const bf16x8 A = *reinterpret_cast<const bf16x8*>(u_lds + ln * kRow + kb + 8 * s);
                    accA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, bA, accA, 0, 0, 0);
                    accX = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, bX, accX, 0, 0, 0);
                }
            }
        } else {
#pragma unroll 4
            for (int k4 = 0; k4 < BS / 2; k4 += 4) {
                const int kb = kh * (BS / 2) + k4;
                const float4 bA = *reinterpret_cast<const float4*>(war + kb);
                const float4 bX = *reinterpret_cast<const float4*>(wxr + kb);
                const float4 A = *reinterpret_cast<const float4*>(u_lds + ln * kRow + kb);
                const float a4[4] = {A.x, A.y, A.z, A.w};
                const float ba4[4] = {bA.x, bA.y, bA.z, bA.w}, bx4[4] = {bX.x, bX.y, bX.z, bX.w};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    accA = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[s], ba4[s], accA, 0, 0, 0);
                    accX = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[s], bx4[s], accX, 0, 0, 0);
                }
            }
        }
    }

    // ---- gate math, state update, output ----
    const float lam = a.lambda[ch];
    const float sp = softplus_neg(lam);
    const float bia = a.ba ? S::get(static_cast<const ST*>(a.ba), ch) : 0.0f;
    const float bix = a.bx ? S::get(static_cast<const ST*>(a.bx), ch) : 0.0f;
    const float nba = -bia * kLog2e, nbx = -bix * kLog2e;
    const float ikc = gate_ikc(sp), kcn = -8.0f * sp;
    const ST* __restrict__ y = static_cast<const ST*>(a.y);
    ST* __restrict__ out = static_cast<ST*>(a.out);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int m = mfma_d_row(lane, j);
        const int n = n0 + m;
        if (n >= N) continue;
        float u;
        if constexpr (kBf) u = bf2f(u_lds[m * kRow + ncol]);
        else u = u_lds[m * kRow + ncol];
        const GateOut g = kBf ? gate_fast(accA[j], accX[j], nba, nbx, ikc, u)
                              : gate_precise(accA[j], accX[j], bia, bix, kcn, u);
        float* hp = a.h + (size_t)n * D + ch;
        const float hn = __builtin_fmaf(g.a, *hp, g.v);
        *hp = hn;
        const float yf = S::get(y, (size_t)n * a.ld_y + ch);
        const float gl = kBf ? gelu_fast(yf) : gelu_precise(yf);
        S::put(out, (size_t)n * a.ld_out + ch, hn * gl);
    }
}

// bf16 storage: the same step with every long-latency load issued up front and none of
// them under a branch.  A load guarded by `n < N` whose value is converted inside the guard
// makes the compiler wait for it there, so each guarded load would cost a full memory round
// trip; here rows past N are clamped to row N-1 (read, never written) and optional operands
// are selected after an unconditional load.  Wave w (of BS/32) owns output channels
// [32w, 32w+32) of the head: one 32x32 MFMA tile per gate, B fragments of all K steps in
// 128 VGPRs.  Order of issue: conv window + x_t, gate weights, then (after the conv) h and y;
// the conv waits only for the first group, the MFMAs for the second, the gate math for the third.
template <int BS>
__global__ void __launch_bounds__(2 * BS) decode_bf16_kernel(DecodeArgs a) {
    constexpr int kThreads = 2 * BS;
    constexpr int kChunks = BS / 8;              // 8-channel chunks of the head
    constexpr int kGroups = kThreads / kChunks;  // 16 sequence groups
    constexpr int kPer = 32 / kGroups;           // sequences per conv thread (2)
    constexpr int kRow = BS + 8;
    constexpr int kKSteps = BS / 16;
    __shared__ __attribute__((aligned(16))) uint16_t u_lds[32 * kRow];

    const int tid = threadIdx.x;
    // Placement: workgroups are dealt to the 8 XCDs round-robin.  Slots are numbered XCD by XCD
    // and walked head-major over (head, tile), so the tiles of one head share an XCD and its
    // gate weights are fetched into that XCD's L2 once per step.
    const unsigned G = gridDim.x, bid = blockIdx.x;
    const unsigned xcd = bid & 7u, jx = bid >> 3, per = G >> 3, rem = G & 7u;
    const unsigned slot = xcd * per + min(xcd, rem) + jx;
    const unsigned n_tiles = (unsigned)((a.N + 31) / 32);
    const int head = (int)(slot / n_tiles);
    const int n0 = (int)(slot % n_tiles) * 32;
    const int N = a.N;
    const size_t D = (size_t)a.D;
    uint16_t* __restrict__ cs = static_cast<uint16_t*>(a.conv_state);
    const uint16_t* __restrict__ xg = static_cast<const uint16_t*>(a.x);
    const int wv = tid >> 6, lane = tid & 63, ln = lane & 31, kh = lane >> 5;

    // ---- group 1: conv taps, bias, window and x_t of this thread's (sequence, chunk) pairs ----
    const int cg = tid % kChunks, sg = tid / kChunks;
    const size_t c0 = (size_t)head * BS + cg * 8;
    const uint4* cwp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.conv_w) + c0 * 4);
    const uint4 cw0 = cwp[0], cw1 = cwp[1], cw2 = cwp[2], cw3 = cwp[3];
    const bool has_cb = a.conv_b != nullptr;
    const uint4 cbv = *reinterpret_cast<const uint4*>(
        has_cb ? static_cast<const uint16_t*>(a.conv_b) + c0 : static_cast<const uint16_t*>(a.conv_w) + c0 * 4);
    uint4 s0[kPer], s1[kPer], s2[kPer], xt[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int n = min(n0 + sg * kPer + k, N - 1);
        const uint16_t* row = cs + (size_t)n * 3 * D + c0;
        s0[k] = *reinterpret_cast<const uint4*>(row);
        s1[k] = *reinterpret_cast<const uint4*>(row + D);
        s2[k] = *reinterpret_cast<const uint4*>(row + 2 * D);
        xt[k] = *reinterpret_cast<const uint4*>(xg + (size_t)n * a.ld_x + c0);
    }
    // ---- group 2: gate weights of this wave's 32 output channels, all K steps, both gates ----
    const int ncol = 32 * wv + ln;
    const size_t chn = (size_t)head * BS + ncol;
    bf16x8 wA[kKSteps], wX[kKSteps];
    {
        const uint16_t* war = static_cast<const uint16_t*>(a.wa) + chn * BS;
        const uint16_t* wxr = static_cast<const uint16_t*>(a.wx) + chn * BS;
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
            const int kb = 64 * (kk >> 2) + 32 * kh + 8 * (kk & 3);
            wA[kk] = *reinterpret_cast<const bf16x8*>(war + kb);
            wX[kk] = *reinterpret_cast<const bf16x8*>(wxr + kb);
        }
    }
    // ---- conv over [window, x_t]; shift the window in place (rows n < N only) ----
    {
        float w[4][8], cb[8];
        const uint32_t* q[4] = {&cw0.x, &cw1.x, &cw2.x, &cw3.x};
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // taps of channel c0 + 2 qq + (e >> 2), tap e & 3
                const uint32_t wd = q[qq][e >> 1];
                w[e & 3][2 * qq + (e >> 2)] = (e & 1) ? bf_hi(wd) : bf_lo(wd);
            }
        const uint32_t* qb = &cbv.x;
#pragma unroll
        for (int e = 0; e < 8; ++e) cb[e] = has_cb ? ((e & 1) ? bf_hi(qb[e >> 1]) : bf_lo(qb[e >> 1])) : 0.0f;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int m = sg * kPer + k;
            const int n = n0 + m;
            const uint32_t* q0 = &s0[k].x;
            const uint32_t* q1 = &s1[k].x;
            const uint32_t* q2 = &s2[k].x;
            const uint32_t* q3 = &xt[k].x;
            float u[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v0 = (e & 1) ? bf_hi(q0[e >> 1]) : bf_lo(q0[e >> 1]);
                const float v1 = (e & 1) ? bf_hi(q1[e >> 1]) : bf_lo(q1[e >> 1]);
                const float v2 = (e & 1) ? bf_hi(q2[e >> 1]) : bf_lo(q2[e >> 1]);
                const float v3 = (e & 1) ? bf_hi(q3[e >> 1]) : bf_lo(q3[e >> 1]);
                float acc = __builtin_fmaf(w[0][e], v0, cb[e]);
                acc = __builtin_fmaf(w[1][e], v1, acc);
                acc = __builtin_fmaf(w[2][e], v2, acc);
                u[e] = __builtin_fmaf(w[3][e], v3, acc);
            }
            *reinterpret_cast<uint4*>(u_lds + m * kRow + cg * 8) =
                make_uint4(pack2bf(u[0], u[1]), pack2bf(u[2], u[3]), pack2bf(u[4], u[5]), pack2bf(u[6], u[7]));
            if (n < N) {
                uint16_t* row = cs + (size_t)n * 3 * D + c0;
                *reinterpret_cast<uint4*>(row) = s1[k];
                *reinterpret_cast<uint4*>(row + D) = s2[k];
                *reinterpret_cast<uint4*>(row + 2 * D) = xt[k];
            }
        }
    }
    // ---- group 3 (issued once the conv registers are free; in flight during the MFMAs):
    // h, y of this lane's 16 (sequence, channel) elements and the gate constants ----
    float hv[16];
    uint16_t yv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int n = min(n0 + mfma_d_row(lane, j), N - 1);
        hv[j] = a.h[(size_t)n * D + chn];
        yv[j] = static_cast<const uint16_t*>(a.y)[(size_t)n * a.ld_y + chn];
    }
    const float lam = a.lambda[chn];
    const uint16_t* bap = static_cast<const uint16_t*>(a.ba);
    const uint16_t* bxp = static_cast<const uint16_t*>(a.bx);
    const uint16_t bav = (bap ? bap : static_cast<const uint16_t*>(a.wa))[bap ? chn : 0];
    const uint16_t bxv = (bxp ? bxp : static_cast<const uint16_t*>(a.wx))[bxp ? chn : 0];

    __syncthreads();

    // ---- gate pre-activations of the 32 sequences on MFMA ----
    f32x16 accA, accX;
#pragma unroll
    for (int e = 0; e < 16; ++e) { accA[e] = 0.0f; accX[e] = 0.0f; }
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
        const int kb = 64 * (kk >> 2) + 32 * kh + 8 * (kk & 3);
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(u_lds + ln * kRow + kb);
        accA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wA[kk], accA, 0, 0, 0);
        accX = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wX[kk], accX, 0, 0, 0);
    }

    // ---- gates, state update, output ----
    const float nba = bap ? -bf2f(bav) * kLog2e : 0.0f;
    const float nbx = bxp ? -bf2f(bxv) * kLog2e : 0.0f;
    const float ikc = gate_ikc(softplus_neg(lam));
    uint16_t* __restrict__ out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int m = mfma_d_row(lane, j);
        const int n = n0 + m;
        const float u = bf2f(u_lds[m * kRow + ncol]);
        const GateOut g = gate_fast(accA[j], accX[j], nba, nbx, ikc, u);
        const float hn = __builtin_fmaf(g.a, hv[j], g.v);
        const float o = hn * gelu_fast(bf2f(yv[j]));
        if (n < N) {
            a.h[(size_t)n * D + chn] = hn;
            out[(size_t)n * a.ld_out + chn] = f2bf(o);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Split decode (used when the caller passes a workspace of N x D storage elements for u).
// The fused kernel above must give each (32 sequences, head) workgroup all of the head's
// gate weights (256 KB at bs = 256), pulled through one CU on every step; that bounds the
// step.  Split in two passes, the work of a head spreads over bs/32 workgroups per 64
// sequences, each pulling only its 32 channels' weights.
// ---------------------------------------------------------------------------------------

// Workspace layout of u between the two passes of the split step: in the order the gate pass's
// MFMA B operands read it.  For a block of 16 sequences, a head and a K step of 32 inputs, one
// contiguous 1 KB block holds 64 lanes x 8 inputs: lane (g, l) = 16 g + l holds inputs
// 32 s + 8 g .. + 7 of sequence 16 nb + l.  Offset (in elements) of sequence n, input chunk c0:
__device__ __forceinline__ size_t u_frag_offset(size_t n, size_t c0, int bs, int H) {
    const size_t head = c0 / (size_t)bs, k0 = c0 % (size_t)bs;
    const size_t s = k0 / 32, g = (k0 % 32) / 8;
    return ((((n / 16) * (size_t)H + head) * (size_t)(bs / 32) + s) * 64 + g * 16 + n % 16) * 8;
}

// Pass 1 of the split step: u = conv([window, x_t]) for 8 channels of one sequence per thread,
// written to the workspace in the storage dtype (nearest-even, as the fused step rounds it) in
// the order above, and the window shifted in place (elementwise: no thread reads what another
// writes).  A wave covers one 1 KB block of that order (16 sequences x 32 channels of one head:
// lane = 16 * (8-channel group) + sequence), so each of its u stores writes one whole block
// instead of sixteen-byte pieces of blocks that other workgroups complete; the four waves of a
// workgroup take neighbouring 32-channel slices, so the window and x rows they read and write
// come in whole 256-byte pieces per sequence.
template <typename ST>
__global__ void __launch_bounds__(256) decode_conv_kernel(DecodeArgs a) {
    using S = Store<ST>;
    const unsigned i = blockIdx.x * blockDim.x + threadIdx.x;
    const unsigned blk = i >> 6, lane = i & 63u;
    const unsigned nslice = (unsigned)a.D >> 5;   // 32-channel slices of all heads
    const unsigned g16 = blk / nslice;            // group of 16 sequences
    const int n_ = (int)(g16 * 16u + (lane & 15u));
    if (n_ >= a.N) return;
    const size_t D = (size_t)a.D, n = (size_t)n_;
    const size_t c0 = (size_t)(blk - g16 * nslice) * 32 + (size_t)(lane >> 4) * 8;
    float w[32], cb[8];
    const ST* cw = static_cast<const ST*>(a.conv_w) + c0 * 4;  // [channel][tap]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float t[8];
        S::load8(cw + 8 * q, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[8 * q + e] = t[e];
    }
    if (a.conv_b) S::load8(static_cast<const ST*>(a.conv_b) + c0, cb);
    else {
#pragma unroll
        for (int e = 0; e < 8; ++e) cb[e] = 0.0f;
    }
    float s0[8], s1[8], s2[8], xt[8];
    ST* cs = static_cast<ST*>(a.conv_state) + n * 3 * D + c0;
    S::load8(cs, s0);
    S::load8(cs + D, s1);
    S::load8(cs + 2 * D, s2);
    S::load8(static_cast<const ST*>(a.x) + n * (size_t)a.ld_x + c0, xt);
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // tap j multiplies x_{t-3+j}: the window holds x_{t-3}, x_{t-2}, x_{t-1}
        float acc = __builtin_fmaf(w[4 * e + 0], s0[e], cb[e]);
        acc = __builtin_fmaf(w[4 * e + 1], s1[e], acc);
        acc = __builtin_fmaf(w[4 * e + 2], s2[e], acc);
        u[e] = __builtin_fmaf(w[4 * e + 3], xt[e], acc);
    }
    // (blk, lane) is exactly this thread's place in the fragment order: u_frag_offset(n, c0)
    S::store8(static_cast<ST*>(a.u_ws) + ((size_t)blk * 64 + lane) * 8, u);
    // the stored values round-trip exactly (bf16 -> fp32 -> bf16)
    S::store8(cs, s1);
    S::store8(cs + D, s2);
    S::store8(cs + 2 * D, xt);
}

// Global -> LDS copy of 16 bytes per lane (buffer load with the LDS bit).
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, int byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, byte_off, 0, 0, 0);
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// LDS-only barrier: the compiler's __syncthreads would also wait for outstanding global loads.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Pass 2 of the split step.  Workgroup = (16 W sequences, head, 32 output channels), W waves of
// 16 sequences each (W = blockDim.x / 64, chosen at launch so that the busiest CU pulls the
// fewest bytes).  The gate weights of the 32 channels (32 rows of each gate, all BS inputs)
// are copied once into LDS and shared by the W waves.  Each wave forms the transposed
// products gates^T = W u^T with 16x16x32 MFMAs: operand A = weight rows from LDS (16 channels),
// operand B = the u rows of its 16 sequences loaded straight from the workspace into VGPRs, so
// the result tile holds 4 consecutive channels of one sequence per lane; h, y and out then move
// as 16- and 8-byte vectors with no LDS round trip.  The gate parameters of the 32 channels
// (Lambda and the two biases) arrive in LDS with the weights; wave 0 turns them into the
// per-channel constants (nb_a, nb_x, 1/kc) beside its MFMAs and shares them through LDS.
template <int BS>
__global__ void __launch_bounds__(512) decode_gate_kernel(DecodeArgs a) {
    constexpr int kKSteps = BS / 32;         // K steps of 32 inputs
    constexpr int kRowB = BS * 2;            // bytes of one weight row
    constexpr int kCB = BS / 32;             // 32-channel blocks per head
    constexpr int kBlocks = 64 * kRowB / 1024;  // 1024-byte copies (16 bytes per lane) of the weights
    // rows 0..31: gate a weights of the 32 channels, rows 32..63: gate x.  The 16-byte chunk at
    // position p of row r holds input chunk p ^ (r & 15), so the 16 rows read by one A fragment
    // fall on distinct banks.
    __shared__ __attribute__((aligned(16))) uint16_t w_lds[64 * BS];
    __shared__ __attribute__((aligned(16))) float k_lds[3 * 32];  // nb_a, nb_x, 1/kc by channel
    // h of each wave's 16 sequences x 32 channels, moved as whole 128-byte rows; the 16-byte
    // chunk at position p of row r holds channels 4 (p ^ (r & 7)) .. + 3, so the MFMA-layout
    // accesses below (16 rows, one chunk each) spread over the banks
    __shared__ __attribute__((aligned(16))) float h_lds[8 * 16 * 32];
    // Lambda (128 bytes), gate a bias, gate x bias (64 bytes each) of the 32 channels; each copy
    // instruction fills 1024 bytes, the lanes past the data repeating it
    __shared__ __attribute__((aligned(16))) unsigned char p_lds[3 * 1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = (int)(blockDim.x >> 6);  // waves, 16 sequences each
    const int l16 = lane & 15, g = lane >> 4;
    const int N = a.N;
    const size_t D = (size_t)a.D;
    // Placement: workgroups are dealt to the 8 XCDs round-robin; slots are numbered XCD by XCD
    // and walked head-major, so the workgroups that share a head's weights share an XCD's L2.
    const unsigned G = gridDim.x, bid = blockIdx.x;
    const unsigned xcd = bid & 7u, jx = bid >> 3, per = G >> 3, rem = G & 7u;
    const unsigned slot = xcd * per + min(xcd, rem) + jx;
    const unsigned n_blocks = (unsigned)((N + 16 * nw - 1) / (16 * nw));
    const int head = (int)(slot / (n_blocks * kCB));
    const unsigned rs = slot % (n_blocks * kCB);
    const int n0 = (int)(rs / kCB) * 16 * nw;
    const int cw0 = (int)(rs % kCB) * 32;
    // a wave whose 16 sequences all lie past N loads and stores nothing (it still copies its
    // share of the weights and meets both barriers); wave 0 is always live
    const bool wave_live = n0 + 16 * wv < N;
    const int nq = n0 + 16 * wv + l16;  // this lane's sequence
    const bool live = nq < N;
    const size_t ns = (size_t)min(nq, N - 1);  // rows past N repeat row N-1 and are not stored
    const size_t cbase = (size_t)head * BS + cw0;

    // 0. gate parameters of the 32 channels -> LDS (wave 0; an absent bias is not copied)
    if (wv == 0) {
        copy16_to_lds(make_rsrc(a.lambda + cbase), p_lds, 16 * (lane & 7));
        if (a.ba) copy16_to_lds(make_rsrc(static_cast<const uint16_t*>(a.ba) + cbase), p_lds + 1024, 16 * (lane & 3));
        if (a.bx) copy16_to_lds(make_rsrc(static_cast<const uint16_t*>(a.bx) + cbase), p_lds + 2048, 16 * (lane & 3));
    }

    // 1. weights -> LDS; each copy instruction fills 1024 / kRowB whole rows of one gate
    {
        const uint16_t* wa = static_cast<const uint16_t*>(a.wa) + cbase * BS;
        const uint16_t* wx = static_cast<const uint16_t*>(a.wx) + cbase * BS;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(wa), rx = make_rsrc(wx);
        for (int blk = wv; blk < kBlocks; blk += nw) {  // 1024-byte block of w_lds
            const int o = blk * 1024 + lane * 16;       // this lane's LDS byte offset
            const int r = o / kRowB, p = (o % kRowB) / 16;
            const int off = ((r & 31) * BS + 8 * (p ^ (r & 15))) * 2;
            copy16_to_lds(blk * 1024 < 32 * kRowB ? ra : rx, w_lds + blk * 512, off);
        }
    }
    // 2. operand B: the u row of this lane's sequence, K-slice g of every K step
    bf16x8 ub[kKSteps];
    uint2 yv[2], uv[2];
    float* const hw = h_lds + wv * 512;  // this wave's h rows
    if (wave_live) {
        // h rows -> LDS, 8 rows per copy (rows past N repeat row N-1 and are not stored)
        const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.h + (size_t)(n0 + 16 * wv) * D + cbase);
        const int last_row = N - 1 - (n0 + 16 * wv);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int r = 8 * q + (lane >> 3), pch = lane & 7;
            const int off = (min(r, last_row) * (int)D + 4 * (pch ^ (r & 7))) * 4;
            copy16_to_lds(rh, hw + 256 * q, off);
        }
        // one contiguous 1 KB block per K step (see u_frag_offset); this wave's 16 sequences are
        // one block of 16
        const uint16_t* ur = static_cast<const uint16_t*>(a.u_ws) +
                             ((((size_t)(n0 / 16 + wv) * a.H + head) * kKSteps) * 64 + lane) * 8;
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) ub[s] = *reinterpret_cast<const bf16x8*>(ur + 512 * s);
        // 3. elementwise operands of channels cbase + 16 t + 4 g + (0..3), t = 0, 1
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const size_t c = cbase + 16 * t + 4 * g;
            yv[t] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.y) + ns * (size_t)a.ld_y + c);
            // inputs cw0 + 16 t + 4 g .. + 3 of this lane's sequence: K step cw0 / 32 (the block the
            // B operand of that step came from), lane group 2 t + g / 2, elements 4 (g & 1) ..
            uv[t] = *reinterpret_cast<const uint2*>(
                static_cast<const uint16_t*>(a.u_ws) +
                ((((size_t)(n0 / 16 + wv) * a.H + head) * kKSteps + cw0 / 32) * 64 +
                 (2 * t + (g >> 1)) * 16 + l16) * 8 + 4 * (g & 1));
        }
    }
    wait_vmem_all();  // this wave's copies and loads have landed
    lds_barrier();    // ... and every wave's copies

    // 4. gate pre-activations: acc[q] rows = channels 16 (q & 1) + (0..15) of gate q >> 1,
    //    columns = the wave's 16 sequences; lane holds rows 4 g + (0..3) of column l16
    f32x4 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (wave_live) {
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 16 * q + l16;
                const bf16x8 A = *reinterpret_cast<const bf16x8*>(w_lds + r * BS + 8 * ((4 * s + g) ^ l16));
                acc[q] = mfma16(A, ub[s], acc[q]);
            }
        }
    }

    // gate constants of channel cbase + lane (wave 0), from hardware exp2/log2/rcp: a few ulp
    // from the library forms of the fused step, and short enough that the other waves hardly
    // wait for them at the barrier below
    if (wv == 0 && lane < 32) {
        const float lam = reinterpret_cast<const float*>(p_lds)[lane];
        const uint16_t* pb = reinterpret_cast<const uint16_t*>(p_lds + 1024);
        k_lds[lane] = a.ba ? -bf2f(pb[lane]) * kLog2e : 0.0f;
        k_lds[32 + lane] = a.bx ? -bf2f(pb[512 + lane]) * kLog2e : 0.0f;
        k_lds[64 + lane] = gate_ikc_fast(softplus_neg_fast(lam));
    }
    lds_barrier();  // the last barrier
    if (!wave_live) return;
    float4 ka[2], kx[2], kk[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        ka[t] = *reinterpret_cast<const float4*>(k_lds + 16 * t + 4 * g);
        kx[t] = *reinterpret_cast<const float4*>(k_lds + 32 + 16 * t + 4 * g);
        kk[t] = *reinterpret_cast<const float4*>(k_lds + 64 + 16 * t + 4 * g);
    }

    // 5. gates, state update, output
    float4* const hq = reinterpret_cast<float4*>(hw);
    float4 hv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) hv[t] = hq[l16 * 8 + ((4 * t + g) ^ (l16 & 7))];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float ua[4] = {bf_lo(uv[t].x), bf_hi(uv[t].x), bf_lo(uv[t].y), bf_hi(uv[t].y)};
        const float ya[4] = {bf_lo(yv[t].x), bf_hi(yv[t].x), bf_lo(yv[t].y), bf_hi(yv[t].y)};
        const float hs[4] = {hv[t].x, hv[t].y, hv[t].z, hv[t].w};
        const float nba[4] = {ka[t].x, ka[t].y, ka[t].z, ka[t].w};
        const float nbx[4] = {kx[t].x, kx[t].y, kx[t].z, kx[t].w};
        const float ikc[4] = {kk[t].x, kk[t].y, kk[t].z, kk[t].w};
        float hn[4], o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const GateOut gt = gate_fast(acc[t][i], acc[2 + t][i], nba[i], nbx[i], ikc[i], ua[i]);
            hn[i] = __builtin_fmaf(gt.a, hs[i], gt.v);
            o[i] = hn[i] * gelu_fast(ya[i]);
        }
        hq[l16 * 8 + ((4 * t + g) ^ (l16 & 7))] = make_float4(hn[0], hn[1], hn[2], hn[3]);
        if (live) {
            const size_t c = cbase + 16 * t + 4 * g;
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + ns * (size_t)a.ld_out + c) =
                make_uint2(pack2bf(o[0], o[1]), pack2bf(o[2], o[3]));
        }
    }
    // new h back to memory as whole rows (the wave's own LDS region: its LDS accesses are in order)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = 8 * q + (lane >> 3), pch = lane & 7;
        const float4 v = hq[r * 8 + pch];
        if (n0 + 16 * wv + r < N)
            *reinterpret_cast<float4*>(a.h + (size_t)(n0 + 16 * wv + r) * D + cbase + 4 * (pch ^ (r & 7))) = v;
    }
}

// conv outputs for a block of kConvTB tokens of one (sequence, 8-channel chunk); reads the old
// window.  All input rows of the block (3 before it, kConvTB in it) are loaded before any is
// used, so a thread has one memory round trip, not one per token.
template <typename ST> struct ConvBlock { static constexpr int kTB = 16; };  // bf16: 19 raw rows = 76 VGPRs
template <> struct ConvBlock<float> { static constexpr int kTB = 8; };       // fp32: 11 raw rows = 88 VGPRs

template <typename ST>
__global__ void __launch_bounds__(256) conv_out_kernel(ConvArgs a) {
    using S = Store<ST>;
    constexpr int kTB = ConvBlock<ST>::kTB;
    constexpr int kRows = kTB + 3;
    constexpr int kWords = 8 * (int)sizeof(ST) / 16;  // 16-byte words per 8-element row chunk
    const int chunks = a.D / 8;
    const int tblocks = (a.T + kTB - 1) / kTB;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (size_t)a.N * chunks * tblocks) return;
    const int cg = (int)(gid % chunks);
    const int tb = (int)((gid / chunks) % tblocks);
    const int n = (int)(gid / ((size_t)chunks * tblocks));
    const size_t D = (size_t)a.D, c0 = (size_t)cg * 8;
    const ST* x = static_cast<const ST*>(a.x);
    const ST* cs = static_cast<const ST*>(a.conv_state);
    const int tbeg = tb * kTB;
    // rows tbeg-3 .. tbeg+kTB-1: before token 0 from the window, past T-1 the row T-1 again
    // (those outputs are not stored)
    uint4 raw[kRows][kWords];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int t = tbeg - 3 + r;
        const ST* src = t >= 0 ? x + ((size_t)n * a.T + min(t, a.T - 1)) * D + c0
                               : cs + ((size_t)n * 3 + 3 + t) * D + c0;
#pragma unroll
        for (int q = 0; q < kWords; ++q) raw[r][q] = reinterpret_cast<const uint4*>(src)[q];
    }
    float w[4][8], cb[8];
    {
        float tmp[8];
        const ST* cw = static_cast<const ST*>(a.conv_w) + c0 * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            S::load8(cw + 8 * q, tmp);
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e & 3][2 * q + (e >> 2)] = tmp[e];
        }
    }
    if (a.conv_b) S::load8(static_cast<const ST*>(a.conv_b) + c0, cb);
    else {
#pragma unroll
        for (int e = 0; e < 8; ++e) cb[e] = 0.0f;
    }
    auto widen = [&](int r, float (&v)[8]) { S::load8(reinterpret_cast<const ST*>(&raw[r][0]), v); };
    float r0[8], r1[8], r2[8];
    widen(0, r0);
    widen(1, r1);
    widen(2, r2);
    ST* o = static_cast<ST*>(a.conv_out);
#pragma unroll
    for (int k = 0; k < kTB; ++k) {
        float xt[8], u[8];
        widen(k + 3, xt);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = __builtin_fmaf(w[0][e], r0[e], cb[e]);
            acc = __builtin_fmaf(w[1][e], r1[e], acc);
            acc = __builtin_fmaf(w[2][e], r2[e], acc);
            u[e] = __builtin_fmaf(w[3][e], xt[e], acc);
            r0[e] = r1[e];
            r1[e] = r2[e];
            r2[e] = xt[e];
        }
        if (tbeg + k < a.T) S::store8(o + ((size_t)n * a.T + tbeg + k) * D + c0, u);
    }
}

// new window = the last three of [old window, x_new] (each element read and written by one thread)
template <typename ST>
__global__ void conv_state_kernel(ConvArgs a) {
    using S = Store<ST>;
    const int chunks = a.D / 8;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (size_t)a.N * chunks) return;
    const int cg = (int)(gid % chunks);
    const int n = (int)(gid / chunks);
    const size_t D = (size_t)a.D, c0 = (size_t)cg * 8;
    ST* cs = static_cast<ST*>(a.conv_state);
    const ST* x = static_cast<const ST*>(a.x);
    float v[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int t = a.T - 3 + j;
        if (t >= 0) S::load8(x + ((size_t)n * a.T + t) * D + c0, v[j]);
        else S::load8(cs + ((size_t)n * 3 + 3 + t) * D + c0, v[j]);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) S::store8(cs + ((size_t)n * 3 + j) * D + c0, v[j]);
}

}  // namespace

// Waves (16 sequences each) per workgroup of the gate pass.  Each workgroup pulls one weight
// slice (64 rows of bs inputs) and, per live wave, 16 u rows plus the wave's h, y and out
// (about 14 bytes per element); the choice minimises the bytes of the busiest CU, i.e.
// ceil(workgroups / CUs) times the bytes of one workgroup, preferring fewer waves on ties.
static int gate_waves(int N, int H, int bs, int ncu) {
    int best = 1;
    double best_cost = 0.0;
    for (int nw = 1; nw <= 8; ++nw) {
        const long long blocks = (N + 16 * nw - 1) / (16 * nw);
        const long long wgs = blocks * H * (bs / 32);
        const int live = min(nw, (N + 15) / 16);
        const double per_wg = 128.0 * bs + live * (32.0 * bs + 16.0 * 32.0 * 14.0);
        const double cost = (double)((wgs + ncu - 1) / ncu) * per_wg;
        if (nw == 1 || cost < best_cost) {
            best = nw;
            best_cost = cost;
        }
    }
    return best;
}

constexpr int kConvBlock = 256;  // threads per workgroup of the conv pass

hipError_t launch_decode(const DecodeArgs& a, int dtype, int bs, hipStream_t s) {
    const dim3 grid((a.N + 31) / 32, a.H);
    // the split form's conv pass indexes its threads (16-sequence group, 32-channel slice,
    // lane) in 32 bits; beyond that (some 6.7 million sequences at D = 2560) the fused kernel runs
    const size_t nc = (size_t)((a.N + 15) / 16) * (size_t)(a.D / 32) * 64;
    if (dtype == 1 && a.u_ws != nullptr && nc < ((size_t)1 << 31)) {
        // split: conv pass over (sequence, 8-channel chunk), then the gate pass
        hipLaunchKernelGGL((decode_conv_kernel<uint16_t>),
                           dim3((unsigned)((nc + kConvBlock - 1) / kConvBlock)), dim3(kConvBlock), 0, s, a);
        const int nw = gate_waves(a.N, a.H, bs, device_cu_count());
        const unsigned g2 = (unsigned)(((a.N + 16 * nw - 1) / (16 * nw)) * a.H * (bs / 32));
        if (bs == 256) hipLaunchKernelGGL((decode_gate_kernel<256>), dim3(g2), dim3(64 * nw), 0, s, a);
        else hipLaunchKernelGGL((decode_gate_kernel<128>), dim3(g2), dim3(64 * nw), 0, s, a);
    } else if (dtype == 1) {
        const dim3 grid1((unsigned)(((a.N + 31) / 32) * a.H));  // (tile, head) placed per XCD
        if (bs == 256) hipLaunchKernelGGL((decode_bf16_kernel<256>), grid1, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((decode_bf16_kernel<128>), grid1, dim3(256), 0, s, a);
    } else {
        if (bs == 256) hipLaunchKernelGGL((decode_kernel<256, float>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((decode_kernel<128, float>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_conv_update(const ConvArgs& a, int dtype, hipStream_t s) {
    const int chunks = a.D / 8;
    if (a.conv_out != nullptr && a.T > 0) {
        const int tb = dtype == 1 ? ConvBlock<uint16_t>::kTB : ConvBlock<float>::kTB;
        const size_t n = (size_t)a.N * chunks * ((a.T + tb - 1) / tb);
        const dim3 grid((unsigned)((n + 255) / 256));
        if (dtype == 1) hipLaunchKernelGGL(conv_out_kernel<uint16_t>, grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(conv_out_kernel<float>, grid, dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t n = (size_t)a.N * chunks;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dtype == 1) hipLaunchKernelGGL(conv_state_kernel<uint16_t>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(conv_state_kernel<float>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rglru
