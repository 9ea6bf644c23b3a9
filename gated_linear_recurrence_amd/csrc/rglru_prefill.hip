// Prefill kernel: the recurrent block's temporal-mixing path over T tokens as a
// time-segmented scan (page "Gemma 詳解：RecurrentGemma 架構", section "含遞迴區塊的殘差區塊":
// conv(k=4) -> RG-LRU on one branch, GELU-tanh on the other, elementwise product).
//
// One workgroup owns one (sequence b, gate head, 64-token segment) unit, taken in ticket order
// from an atomic counter so that every unit it may wait on has already started.
//   1. conv: each thread convolves 8 channels x 4 tokens (fp32 FMAs) and writes u to LDS.
//   2. gates: wave w computes output channels [32w, 32w+32) of both gates for all 64 tokens
//      with 32x32 MFMA tiles (bf16 inputs, fp32 accumulate; fp32 MFMA for fp32 storage).
//      The tile rows are permuted so that each lane's accumulators hold 32 consecutive
//      tokens of one channel (low half-wave: tokens 0..31, high half-wave: 32..63).
//   3. gate math (fp32) and a sequential scan in registers from a zero state:
//      b_t = a_t b_{t-1} + v_t,  p_t = p_{t-1} a_t; the half-waves' aggregates combine into
//      the segment aggregate (A, B) = (prod a, local state at the segment end).
//   4. carry: decoupled look-back over per-channel 64-bit words (A | status, B) of earlier
//      segments; carries are always folded forward from an inclusive word, so the result
//      does not depend on timing.
//   5. fix-up h_t = b_t + p_t * carry, out_t = h_t * gelu_tanh(y_t), store.
#include <type_traits>

#include "rglru_device.h"
#include "rglru_internal.h"

namespace rglru {

namespace {

constexpr int kWindow = 8;                 // look-back window (words read per poll)
constexpr unsigned kSpinLimit = 1u << 20;  // polls before a carry wait gives up (error flag)
constexpr unsigned long long kNotReady = ~0ull;

// ---- carry words: low 32 bits = A in [0, 1] (bit 31 set = inclusive), high 32 bits = B ----
__device__ __forceinline__ unsigned long long make_word(float A, float B, bool inclusive) {
    const float ac = fminf(fmaxf(A, 0.0f), 1.0f);  // canonical: finite, non-negative
    const unsigned lo = (__float_as_uint(ac) & 0x7fffffffu) | (inclusive ? 0x80000000u : 0u);
    return ((unsigned long long)__float_as_uint(B) << 32) | lo;
}
__device__ __forceinline__ bool w_ready(unsigned long long w) { return (unsigned)w != 0xffffffffu; }
__device__ __forceinline__ bool w_inclusive(unsigned long long w) { return (unsigned)w & 0x80000000u; }
__device__ __forceinline__ float w_A(unsigned long long w) { return __uint_as_float((unsigned)w & 0x7fffffffu); }
__device__ __forceinline__ float w_B(unsigned long long w) { return __uint_as_float((unsigned)(w >> 32)); }

__device__ __forceinline__ unsigned long long ld_word(unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(unsigned long long* p, unsigned long long w) {
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Carry into segment `seg` (> 0) for one channel.  wself points at this segment's word;
// the predecessor's word is wself - wstride.
__device__ float look_back(unsigned long long* wself, size_t wstride, int seg, float A_seg,
                           float B_seg, bool publish_aggregate, unsigned* header) {
    const unsigned long long w1 = ld_word(wself - wstride);
    if (w_ready(w1) && w_inclusive(w1)) return w_B(w1);
    if (publish_aggregate) st_word(wself, make_word(A_seg, B_seg, false));
    const int n = seg < kWindow ? seg : kWindow;
    for (unsigned it = 0;; ++it) {
        unsigned long long win[kWindow];
#pragma unroll
        for (int k = 0; k < kWindow; ++k)
            win[k] = (k < n) ? ld_word(wself - (size_t)(k + 1) * wstride) : kNotReady;
        int kinc = -1;
        bool blocked = false;
#pragma unroll
        for (int k = 0; k < kWindow; ++k) {
            if (kinc < 0 && !blocked) {
                if (!w_ready(win[k])) blocked = true;
                else if (w_inclusive(win[k])) kinc = k;
            }
        }
        if (kinc >= 0) {
            // fold forward from the inclusive word (oldest) to the predecessor (newest)
            float c = 0.0f;
#pragma unroll
            for (int k = kWindow - 1; k >= 0; --k) {
                if (k == kinc) c = w_B(win[k]);
                else if (k < kinc) c = __builtin_fmaf(w_A(win[k]), c, w_B(win[k]));
            }
            return c;
        }
        if (it >= kSpinLimit) {
            atomicOr(&header[1], 1u);
            return __builtin_nanf("");
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// LDS row of token t (0..63): tokens 32..63 have row bits 2..3 flipped so that the MFMA
// A-fragment reads (tokens {t, t+32} in one pass) fall in different bank groups.
__device__ __forceinline__ int lds_row(int t) { return t ^ (((t >> 5) & 1) * 12); }

template <int BS, typename ST>
struct Cfg {
    static constexpr bool kBf = Store<ST>::kBf16;
    static constexpr int kWaves = BS / 32;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kChunks = BS / 8;               // 8-channel chunks per token row
    static constexpr int kTokGroups = kThreads / kChunks; // = 16
    static constexpr int kTokPerThread = kSeg / kTokGroups;
    static constexpr int kRow = kBf ? BS + 8 : BS + 4;    // LDS row stride (elements)
    using Lds = typename std::conditional<kBf, uint16_t, float>::type;
    static_assert(kTokGroups * kTokPerThread == kSeg, "conv tiling");
};

// Fix-up, GELU merge and stores for one lane's 32 tokens.
template <bool kLast, int BS, typename ST>
__device__ __forceinline__ void finish_outputs(const f32x16 (&accB)[2], const f32x16 (&accP)[2],
                                               const ST (&yv)[2][16], float state_in,
                                               ST* __restrict__ out, size_t base, size_t D,
                                               int hh, int nt, int t0, int T,
                                               float* __restrict__ h_last, size_t hidx) {
    using S = Store<ST>;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int tok = 32 * hh + 16 * mt + j;
            if (kLast && tok >= nt) continue;
            const float h = __builtin_fmaf(accP[mt][j], state_in, accB[mt][j]);
            float yf;
            if constexpr (S::kBf16) yf = bf2f(yv[mt][j]);
            else yf = yv[mt][j];
            const float g = S::kBf16 ? gelu_fast(yf) : gelu_precise(yf);
            S::put(out, base + (size_t)(16 * mt + j) * D, h * g);
            if (kLast && h_last != nullptr && t0 + tok == T - 1) h_last[hidx] = h;
        }
    }
}

template <int BS, typename ST>
__global__ void __launch_bounds__(2 * BS, 2) prefill_kernel(PrefillArgs a) {
    using C = Cfg<BS, ST>;
    using S = Store<ST>;
    using L = typename C::Lds;
    constexpr bool kBf = C::kBf;
    constexpr int kRow = C::kRow;

    __shared__ __attribute__((aligned(16))) L u_lds[kSeg * kRow];
    __shared__ unsigned s_ticket;

    const int tid = threadIdx.x;
    if (tid == 0) s_ticket = atomicAdd(&a.header[0], 1u);
    __syncthreads();
    const unsigned ticket = s_ticket;
    const int n_chains = a.B * a.H;
    const int seg = (int)(ticket / (unsigned)n_chains);
    const int chain = (int)(ticket % (unsigned)n_chains);
    const int b = chain / a.H;
    const int head = chain % a.H;
    const int T = a.T;
    const size_t D = (size_t)a.D;
    const int t0 = seg * kSeg;
    const int nt = min(kSeg, T - t0);
    const bool last = (seg == a.S - 1);

    const ST* __restrict__ x = static_cast<const ST*>(a.x);
    const ST* __restrict__ y = static_cast<const ST*>(a.y);
    ST* __restrict__ out = static_cast<ST*>(a.out);

    // ---------------- 1. causal depthwise conv (k = 4) -> u in LDS ----------------
    {
        const int cg = tid % C::kChunks, tg = tid / C::kChunks;
        const int c0 = head * BS + cg * 8;
        const ST* cw = static_cast<const ST*>(a.conv_w) + (size_t)c0 * 4;
        float w[4][8];  // w[j][channel]
        {
            float tmp[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // 32 contiguous weights: channels c0..c0+7, taps 0..3
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
        constexpr int kR = C::kTokPerThread + 3;
        float xr[kR][8];
        const int tbase = tg * C::kTokPerThread;
#pragma unroll
        for (int k = 0; k < kR; ++k) {
            const int tr = t0 + tbase - 3 + k;
            if (tr >= 0 && tr < T) {
                S::load8(x + ((size_t)b * T + tr) * D + c0, xr[k]);
            } else if (tr < 0 && a.conv0 != nullptr) {
                S::load8(static_cast<const ST*>(a.conv0) + ((size_t)b * 3 + 3 + tr) * D + c0, xr[k]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) xr[k][e] = 0.0f;
            }
        }
#pragma unroll
        for (int k = 0; k < C::kTokPerThread; ++k) {
            const int tok = tbase + k;
            float u[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = __builtin_fmaf(w[0][e], xr[k][e], cb[e]);
                acc = __builtin_fmaf(w[1][e], xr[k + 1][e], acc);
                acc = __builtin_fmaf(w[2][e], xr[k + 2][e], acc);
                acc = __builtin_fmaf(w[3][e], xr[k + 3][e], acc);
                u[e] = tok < nt ? acc : 0.0f;
            }
            L* dst = u_lds + lds_row(tok) * kRow + cg * 8;
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

    // ---------------- 2. block-diagonal gate projections on MFMA ----------------
    const int wv = tid >> 6, lane = tid & 63, ln = lane & 31, kh = lane >> 5, hh = lane >> 5;
    const int ncol = wv * 32 + ln;               // output channel within the head
    const size_t ch = (size_t)head * BS + ncol;  // global channel of this lane's accumulators
    // A-fragment row ln of tile mt holds token 32*bit2(ln) + 16*mt + 4*(ln>>3) + (ln&3)
    const int atok = 32 * ((ln >> 2) & 1) + 4 * (ln >> 3) + (ln & 3);
    const int arow0 = lds_row(atok), arow1 = lds_row(atok + 16);
    f32x16 accB[2], accP[2];  // gate sums (a: accB, x: accP), later the scan values b_t, p_t
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        accB[0][e] = 0.0f; accB[1][e] = 0.0f; accP[0][e] = 0.0f; accP[1][e] = 0.0f;
    }
    {
        const ST* war = static_cast<const ST*>(a.wa) + ((size_t)head * BS + ncol) * BS;
        const ST* wxr = static_cast<const ST*>(a.wx) + ((size_t)head * BS + ncol) * BS;
        if constexpr (kBf) {
#pragma unroll
            for (int q4 = 0; q4 < BS / 64; ++q4) {
                // lane supplies K elements [64 q4 + 32 kh, +32): 8 per MFMA step, 4 steps
                const int kb = 64 * q4 + 32 * kh;
                bf16x8 bA[4], bX[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bA[s] = *reinterpret_cast<const bf16x8*>(war + kb + 8 * s);
                    bX[s] = *reinterpret_cast<const bf16x8*>(wxr + kb + 8 * s);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(u_lds + arow0 * kRow + kb + 8 * s);
                    const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(u_lds + arow1 * kRow + kb + 8 * s);
                    accB[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, bA[s], accB[0], 0, 0, 0);
                    accP[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, bX[s], accP[0], 0, 0, 0);
                    accB[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, bA[s], accB[1], 0, 0, 0);
                    accP[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, bX[s], accP[1], 0, 0, 0);
                }
            }
        } else {
            // fp32: 32x32x2 steps; the lane supplies K element kh*BS/2 + kk at step kk
#pragma unroll 4
            for (int k4 = 0; k4 < BS / 2; k4 += 4) {
                const int kb = kh * (BS / 2) + k4;
                const float4 bA = *reinterpret_cast<const float4*>(war + kb);
                const float4 bX = *reinterpret_cast<const float4*>(wxr + kb);
                const float4 A0 = *reinterpret_cast<const float4*>(u_lds + arow0 * kRow + kb);
                const float4 A1 = *reinterpret_cast<const float4*>(u_lds + arow1 * kRow + kb);
                const float a0[4] = {A0.x, A0.y, A0.z, A0.w}, a1[4] = {A1.x, A1.y, A1.z, A1.w};
                const float ba4[4] = {bA.x, bA.y, bA.z, bA.w}, bx4[4] = {bX.x, bX.y, bX.z, bX.w};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    accB[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[s], ba4[s], accB[0], 0, 0, 0);
                    accP[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[s], bx4[s], accP[0], 0, 0, 0);
                    accB[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[s], ba4[s], accB[1], 0, 0, 0);
                    accP[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[s], bx4[s], accP[1], 0, 0, 0);
                }
            }
        }
    }

    // y for this lane's 32 tokens: issue the loads before the gate math and the look-back
    ST yv[2][16];
    const size_t obase = ((size_t)b * T + t0 + 32 * hh) * D + ch;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int tok = 32 * hh + 16 * mt + j;
            yv[mt][j] = (!last || tok < nt) ? y[obase + (size_t)(16 * mt + j) * D] : (ST)0;
        }
    }

    // ---------------- 3. gate math (fp32) and the local scan in registers ----------------
    float psc = 1.0f, bsc = 0.0f;
    {
        const float lam = a.lambda[ch];
        const float sp = softplus_neg(lam);
        const float bia = a.ba ? S::get(static_cast<const ST*>(a.ba), ch) : 0.0f;
        const float bix = a.bx ? S::get(static_cast<const ST*>(a.bx), ch) : 0.0f;
        const float nba = -bia * kLog2e, nbx = -bix * kLog2e;
        const float kc = -8.0f * sp * kLog2e;  // log2(a) = kc * r
        const float kcn = -8.0f * sp;          // ln(a) = kcn * r
        // LDS row of register j (tile mt): 32 hh + 16 mt + 4 ((j>>2) ^ 3 hh) + (j & 3)
        const L* ucol = u_lds + 32 * hh * kRow + ncol;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = 16 * mt + 4 * ((j >> 2) ^ (3 * hh)) + (j & 3);
                float u;
                if constexpr (kBf) u = bf2f(ucol[row * kRow]);
                else u = ucol[row * kRow];
                const GateOut g = kBf ? gate_fast(accB[mt][j], accP[mt][j], nba, nbx, kc, u)
                                      : gate_precise(accB[mt][j], accP[mt][j], bia, bix, kcn, u);
                bsc = __builtin_fmaf(g.a, bsc, g.v);
                psc = psc * g.a;
                accB[mt][j] = bsc;
                accP[mt][j] = psc;
            }
        }
    }
    // segment aggregate: low half-wave (tokens 0..31) then high half-wave (32..63)
    const float p_o = __shfl_xor(psc, 32), b_o = __shfl_xor(bsc, 32);
    const float p_lo = hh ? p_o : psc, b_lo = hh ? b_o : bsc;
    const float p_hi = hh ? psc : p_o, b_hi = hh ? bsc : b_o;
    const float A_seg = p_lo * p_hi;
    const float B_seg = __builtin_fmaf(p_hi, b_lo, b_hi);

    // ---------------- 4. carry from earlier segments ----------------
    float carry = 0.0f;
    {
        const size_t wstride = (size_t)a.B * D;
        unsigned long long* wself = a.words + (size_t)seg * wstride + (size_t)b * D + ch;
        if (hh == 0) {
            if (seg == 0) {
                carry = a.h0 ? a.h0[(size_t)b * D + ch] : 0.0f;
            } else {
                carry = look_back(wself, wstride, seg, A_seg, B_seg, !last, a.header);
            }
            if (!last) st_word(wself, make_word(A_seg, __builtin_fmaf(A_seg, carry, B_seg), true));
            if (seg > 0) st_word(wself - wstride, kNotReady);  // retire the predecessor's word
        }
    }
    carry = __shfl(carry, ln);
    const float state_in = hh ? __builtin_fmaf(p_lo, carry, b_lo) : carry;

    // ---------------- 5. fix-up, GELU merge, store ----------------
    const size_t hidx = (size_t)b * D + ch;
    if (last)
        finish_outputs<true, BS, ST>(accB, accP, yv, state_in, out, obase, D, hh, nt, t0, T,
                                     a.h_last, hidx);
    else
        finish_outputs<false, BS, ST>(accB, accP, yv, state_in, out, obase, D, hh, nt, t0, T,
                                      a.h_last, hidx);

    // conv state after the last token: x~[T-3 .. T-1] (earlier rows from conv0, or zeros)
    if (last && a.conv_last != nullptr) {
        float v[8];
        const int jr = tid / C::kChunks, cg = tid % C::kChunks;
        const bool act = jr < 3;
        if (act) {
            const int tr = T - 3 + jr;
            const size_t c0 = (size_t)head * BS + cg * 8;
            if (tr >= 0) S::load8(x + ((size_t)b * T + tr) * D + c0, v);
            else if (a.conv0 != nullptr)
                S::load8(static_cast<const ST*>(a.conv0) + ((size_t)b * 3 + 3 + tr) * D + c0, v);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.0f;
            }
        }
        __syncthreads();  // conv0 may alias conv_last: every read before any write
        if (act) {
            const size_t c0 = (size_t)head * BS + cg * 8;
            S::store8(static_cast<ST*>(a.conv_last) + ((size_t)b * 3 + jr) * D + c0, v);
        }
    }

    // the last workgroup to finish resets the counters for the next call on this workspace
    if (tid == 0) {
        const unsigned done = atomicAdd(&a.header[2], 1u);
        if (done == (unsigned)a.n_units - 1) {
            atomicExch(&a.header[0], 0u);
            atomicExch(&a.header[2], 0u);
        }
    }
}

// T = 0: state passes through (h_last = h0 or 0, conv_last = conv0 or 0).
template <typename ST>
__global__ void prefill_empty_kernel(PrefillArgs a) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t nd = (size_t)a.B * a.D;
    if (a.h_last && i < nd) a.h_last[i] = a.h0 ? a.h0[i] : 0.0f;
    if (a.conv_last && i < 3 * nd) {
        const ST* c0 = static_cast<const ST*>(a.conv0);
        static_cast<ST*>(a.conv_last)[i] = c0 ? c0[i] : (ST)0;
    }
}

__global__ void workspace_init_kernel(unsigned long long* p, size_t n_words) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_words) p[i] = (i < kWsHeader / 8) ? 0ull : kNotReady;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int bs, hipStream_t s) {
    const dim3 grid(a.n_units);
    if (dtype == 1) {
        if (bs == 256) hipLaunchKernelGGL((prefill_kernel<256, uint16_t>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((prefill_kernel<128, uint16_t>), grid, dim3(256), 0, s, a);
    } else {
        if (bs == 256) hipLaunchKernelGGL((prefill_kernel<256, float>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((prefill_kernel<128, float>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_empty(const PrefillArgs& a, int dtype, hipStream_t s) {
    const size_t n = 3 * (size_t)a.B * a.D;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dtype == 1) hipLaunchKernelGGL(prefill_empty_kernel<uint16_t>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(prefill_empty_kernel<float>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 8;
    const dim3 grid((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(workspace_init_kernel, grid, dim3(256), 0, s,
                       static_cast<unsigned long long*>(ws), n);
    return hipGetLastError();
}

}  // namespace rglru
