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
#include <atomic>
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
// the predecessor's word is wself - wstride and w1 is a value already read from it.  The
// window is read before this segment's aggregate is published so that waiting for the reads
// never waits for that store.
__device__ float look_back(unsigned long long* wself, size_t wstride, int seg, unsigned long long w1,
                           float A_seg, float B_seg, bool publish_aggregate, unsigned* header) {
    if (w_ready(w1) && w_inclusive(w1)) return w_B(w1);
    const int n = seg < kWindow ? seg : kWindow;
    bool published = !publish_aggregate;
    for (unsigned it = 0;; ++it) {
        unsigned long long win[kWindow];
#pragma unroll
        for (int k = 0; k < kWindow; ++k)
            win[k] = (k < n) ? ld_word(wself - (size_t)(k + 1) * wstride) : kNotReady;
        if (!published) {
            st_word(wself, make_word(A_seg, B_seg, false));
            published = true;
        }
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
            atomicOr(&header[kErrWord], 1u);
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

// Generic kernel (fp32 and bf16 storage, exact-precision gate math for fp32); one ticket
// counter over all units.  The bf16 storage path uses prefill_bf16_kernel below.
template <int BS, typename ST>
__global__ void __launch_bounds__(2 * BS) prefill_kernel(PrefillArgs a) {
    using C = Cfg<BS, ST>;
    using S = Store<ST>;
    using L = typename C::Lds;
    constexpr bool kBf = C::kBf;
    constexpr int kRow = C::kRow;

    __shared__ __attribute__((aligned(16))) L u_lds[kSeg * kRow];
    __shared__ unsigned s_ticket;

    const int tid = threadIdx.x;
    if (tid == 0) s_ticket = atomicAdd(&a.header[kTicketWord], 1u);
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
                carry = look_back(wself, wstride, seg, ld_word(wself - wstride), A_seg, B_seg, !last,
                                  a.header);
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
        const unsigned done = atomicAdd(&a.header[kDoneWord], 1u);
        if (done == (unsigned)a.n_units - 1) {
            atomicExch(&a.header[kTicketWord], 0u);
            atomicExch(&a.header[kDoneWord], 0u);
        }
    }
}

// ---------------------------------------------------------------------------------------
// bf16 storage, persistent kernel (the measured path).
//
// One workgroup per CU, pinned to one gate head for its lifetime: each wave keeps the B
// fragments of its 32 output channels of both gate blocks in VGPRs (128 registers), so the
// gate weights are read once per workgroup instead of once per segment.  The workgroup walks
// the head's segments in ticket order (segment-major over the batch) and pipelines them:
//   iteration k:  [conv k: x_k (LDS) -> u (LDS)] [store out_{k-1}] [DMA x_{k+1}, y_{k+1}]
//                 [MFMA k] [gate math + scan k] [carry k] [GELU merge k -> registers]
// x and y reach LDS by direct global->LDS loads (global_load_lds_dwordx4) one segment ahead;
// the outputs of segment k are stored during iteration k+1, after its conv, so no wait on
// the memory counter ever waits for freshly issued stores.
// Placement: the hardware deals workgroups to the 8 XCDs round-robin; consecutive slots of
// one XCD are given to one head, so each XCD's L2 serves few heads.
// ---------------------------------------------------------------------------------------
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffff, 0x00020000);
}

__device__ __forceinline__ float dot2bf(uint32_t w, uint32_t x, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, x), c, false);
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

#ifndef RGLRU_NT256
#define RGLRU_NT256 1
#endif
constexpr int kSchedGroup = 4;  // elements the scheduler may interleave (bounds register use)

template <int BS>
struct PCfg {
    static constexpr int kNT = BS == 256 ? RGLRU_NT256 : 1;  // 32-channel MFMA tiles per wave
    static constexpr int kWaves = BS / (32 * kNT);      // 4 waves: one per SIMD
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kRow = BS + 8;                 // ubuf row stride (bf16 elements)
    static constexpr int kRowB = BS * 2;                // bytes of one head's slice of a token row
    static constexpr int kHalo = 16;                    // xbuf rows before the segment
    static constexpr int kXRows = kSeg + kHalo;         // tokens t0-16 .. t0+63
    static constexpr int kRowsPerInst = 1024 / kRowB;   // one DMA instruction moves 1 KB
    static constexpr int kLanesPerRow = kRowB / 16;
    static constexpr int kXInst = kXRows / kRowsPerInst / kWaves;
    static constexpr int kYInst = kSeg / kRowsPerInst / kWaves;
    static constexpr int kPairs = BS / 2;               // conv: channel pairs ...
    static constexpr int kTokGroups = kThreads / kPairs;  // ... x token groups
    static constexpr int kTok = kSeg / kTokGroups;
    static constexpr int kKSteps = BS / 16;
    static_assert(kXInst * kRowsPerInst * kWaves == kXRows, "x DMA tiling");
    static_assert(kYInst * kRowsPerInst * kWaves == kSeg, "y DMA tiling");
    static_assert(kTokGroups * kTok == kSeg, "conv tiling");
};

// Direct global->LDS copy of one segment's rows of one head: LDS row r receives token
// t0 + first + r of the ticket's sequence, clamped to [0, T-1]; a ticket past the end copies
// the last segment again (harmless).
template <int BS, int kInst>
__device__ __forceinline__ void dma_rows(const char* head_base, unsigned tk, unsigned n_tk, int B,
                                         int T, int rowb, int first, int wv, int dma_r,
                                         uint16_t* lds) {
    using C = PCfg<BS>;
    tk = min(tk, n_tk - 1);
    const int t0 = (int)(tk / (unsigned)B) * kSeg;
    const char* base = head_base + (size_t)(tk % (unsigned)B) * T * rowb;
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
        const int inst = wv * kInst + q;
        const int tr = min(max(t0 + first + inst * C::kRowsPerInst + dma_r, 0), T - 1);
        __builtin_amdgcn_global_load_lds(base + (size_t)tr * rowb, lds + inst * 512, 16, 0, 0);
    }
}

// A copy of v that the compiler cannot see through: values derived from it inside the loop
// are recomputed there instead of being kept live across it (the gate weights already occupy
// half of the register file).
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int BS>
__global__ void __launch_bounds__(PCfg<BS>::kThreads)
prefill_bf16_kernel(PrefillArgs a) {
    using C = PCfg<BS>;
    constexpr int kNT = C::kNT;
    constexpr int kRow = C::kRow;
    __shared__ __attribute__((aligned(16))) uint16_t xbuf[C::kXRows * BS];
    __shared__ __attribute__((aligned(16))) uint16_t ybuf[2][kSeg * BS];
    __shared__ __attribute__((aligned(16))) uint16_t ubuf[kSeg * kRow];
    __shared__ __attribute__((aligned(16))) uint4 conv_tab[BS / 2];   // taps of a channel pair
    __shared__ __attribute__((aligned(8))) float2 convb_tab[BS / 2];  // biases of a channel pair
    __shared__ __attribute__((aligned(16))) float4 gate_tab[BS];      // (nba, nbx, kc, 0) per channel
    __shared__ unsigned s_tk[2];

    const int tid0 = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int B = a.B, T = a.T;
    const size_t D = (size_t)a.D;
    const int rowb = (int)(D * 2);

    // ---- placement: slot -> head ----
    const unsigned G = gridDim.x, bid = blockIdx.x;
    const unsigned xcd = bid & 7u, jx = bid >> 3, per = G >> 3, rem = G & 7u;
    const unsigned slot = xcd * per + min(xcd, rem) + jx;
    const int head = (int)(slot / (unsigned)a.wph);
    unsigned* tctr = a.header + kTicketWord + head;
    const unsigned n_tk = (unsigned)(B * a.S);

    const uint16_t* __restrict__ x = static_cast<const uint16_t*>(a.x);
    const uint16_t* __restrict__ y = static_cast<const uint16_t*>(a.y);

    // ---- per-workgroup tables: conv taps and biases, gate constants of the head's channels ----
    for (int i = tid0; i < BS / 2; i += C::kThreads) {
        const size_t c0 = (size_t)head * BS + 2 * i;
        conv_tab[i] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.conv_w) + c0 * 4);
        float2 cb = make_float2(0.0f, 0.0f);
        if (a.conv_b) {
            const uint32_t bb = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.conv_b) + c0);
            cb = make_float2(bf_lo(bb), bf_hi(bb));
        }
        convb_tab[i] = cb;
    }
    for (int i = tid0; i < BS; i += C::kThreads) {
        const size_t chn = (size_t)head * BS + i;
        const float sp = softplus_neg(a.lambda[chn]);
        const float bia = a.ba ? bf2f(static_cast<const uint16_t*>(a.ba)[chn]) : 0.0f;
        const float bix = a.bx ? bf2f(static_cast<const uint16_t*>(a.bx)[chn]) : 0.0f;
        gate_tab[i] = make_float4(-bia * kLog2e, -bix * kLog2e, -8.0f * sp * kLog2e, 0.0f);
    }
    // gate weights of this wave's channels [cw0, cw0 + 32 kNT), held in registers throughout
    const int cw0 = wv * 32 * kNT;
    bf16x8 wA[kNT][C::kKSteps], wX[kNT][C::kKSteps];
    {
        const int lane = tid0 & 63, ln = lane & 31, kh = lane >> 5;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const size_t chn = (size_t)head * BS + cw0 + 32 * nt + ln;
            const uint16_t* war = static_cast<const uint16_t*>(a.wa) + chn * BS;
            const uint16_t* wxr = static_cast<const uint16_t*>(a.wx) + chn * BS;
#pragma unroll
            for (int kk = 0; kk < C::kKSteps; ++kk) {
                // K order: lane half kh supplies elements [64 q + 32 kh + 8 s, +8) at step 4q + s
                const int kb = 64 * (kk >> 2) + 32 * kh + 8 * (kk & 3);
                wA[nt][kk] = *reinterpret_cast<const bf16x8*>(war + kb);
                wX[nt][kk] = *reinterpret_cast<const bf16x8*>(wxr + kb);
            }
        }
    }
    const char* xseq = reinterpret_cast<const char*>(x + (size_t)head * BS);
    const char* yseq = reinterpret_cast<const char*>(y + (size_t)head * BS);

    // ---- prologue ----
    if (tid0 == 0) {
        s_tk[0] = atomicAdd(tctr, 1u);
        s_tk[1] = atomicAdd(tctr, 1u);
    }
    __syncthreads();
    unsigned cur = s_tk[0], nxt = s_tk[1];
    {
        const int lane = tid0 & 63;
        const char* xh = xseq + 16 * (lane % C::kLanesPerRow);
        const char* yh = yseq + 16 * (lane % C::kLanesPerRow);
        dma_rows<BS, C::kXInst>(xh, cur, n_tk, B, T, rowb, -C::kHalo, wv, lane / C::kLanesPerRow, xbuf);
        dma_rows<BS, C::kYInst>(yh, cur, n_tk, B, T, rowb, 0, wv, lane / C::kLanesPerRow, ybuf[0]);
    }
    wait_vmem_all();
    unsigned it = 0;

    while (cur < n_tk) {
        const int tid = opaque(tid0);
        const int lane = tid & 63, ln = lane & 31, kh = lane >> 5, hh = lane >> 5;
        const int seg = (int)(cur / (unsigned)B), b = (int)(cur % (unsigned)B);
        const int t0 = seg * kSeg;
        const int nt_tok = min(kSeg, T - t0);
        const bool last = (seg == a.S - 1);
        const uint16_t* ycur = ybuf[it & 1];

        // x and y of `cur` have landed: each wave waited for its own DMA (prologue or the
        // previous iteration); the barrier covers every wave
        __syncthreads();
        if (it > 0) nxt = s_tk[0];  // grabbed during the previous iteration, published before the barrier
        if (seg == 0) {
            // tokens -3..-1 come from the carried conv state (or are zero), not from x
            constexpr int kCh = BS / 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (tid < 3 * kCh && a.conv0 != nullptr)
                v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.conv0) +
                                                    ((size_t)b * 3 + tid / kCh) * D + (size_t)head * BS + (tid % kCh) * 8);
            if (tid < 3 * kCh)
                *reinterpret_cast<uint4*>(xbuf + (C::kHalo - 3 + tid / kCh) * BS + (tid % kCh) * 8) = v;
            __syncthreads();
        }

        // ---------------- 1. conv -> u (bf16) in LDS ----------------
        {
            const int cp = tid % C::kPairs;
            const int tg = __builtin_amdgcn_readfirstlane(tid / C::kPairs);
            const uint4 wq = conv_tab[cp];
            const float2 cb = convb_tab[cp];
            const uint32_t* xw = reinterpret_cast<const uint32_t*>(xbuf);
            uint32_t xr[C::kTok + 3];
#pragma unroll
            for (int k = 0; k < C::kTok + 3; ++k)
                xr[k] = xw[(tg * C::kTok + C::kHalo - 3 + k) * C::kPairs + cp];
            uint16_t* ucol = ubuf + 2 * cp;
#pragma unroll
            for (int k = 0; k < C::kTok; ++k) {
                // (x_{t-3}, x_{t-2}) and (x_{t-1}, x_t) of each of the two channels
                const uint32_t p0a = __builtin_amdgcn_perm(xr[k + 1], xr[k], 0x05040100u);
                const uint32_t p0b = __builtin_amdgcn_perm(xr[k + 1], xr[k], 0x07060302u);
                const uint32_t p2a = __builtin_amdgcn_perm(xr[k + 3], xr[k + 2], 0x05040100u);
                const uint32_t p2b = __builtin_amdgcn_perm(xr[k + 3], xr[k + 2], 0x07060302u);
                const float u0 = dot2bf(wq.y, p2a, dot2bf(wq.x, p0a, cb.x));
                const float u1 = dot2bf(wq.w, p2b, dot2bf(wq.z, p0b, cb.y));
                *reinterpret_cast<uint32_t*>(ucol + lds_row(tg * C::kTok + k) * kRow) = pack2bf(u0, u1);
            }
        }
        // conv state after the last token: rows T-3..T-1 are in xbuf now; they are written
        // after the carry wait, which orders the write after segment 0 read conv0 (in place)
        uint4 cl_rows = make_uint4(0, 0, 0, 0);
        constexpr int kClCh = BS / 8;
        const bool cl_act = last && a.conv_last != nullptr && tid < 3 * kClCh;
        if (cl_act)
            cl_rows = *reinterpret_cast<const uint4*>(xbuf + (T - 3 + tid / kClCh - t0 + C::kHalo) * BS +
                                                      (tid % kClCh) * 8);
        __syncthreads();  // u complete; xbuf and ybuf[(it+1)&1] are free

        // ---------------- prefetch the next segment ----------------
        {
            const char* xh = xseq + 16 * (lane % C::kLanesPerRow);
            const char* yh = yseq + 16 * (lane % C::kLanesPerRow);
            dma_rows<BS, C::kXInst>(xh, nxt, n_tk, B, T, rowb, -C::kHalo, wv, lane / C::kLanesPerRow, xbuf);
            dma_rows<BS, C::kYInst>(yh, nxt, n_tk, B, T, rowb, 0, wv, lane / C::kLanesPerRow, ybuf[(it + 1) & 1]);
        }
        unsigned pending = 0;
        if (tid == 0) pending = atomicAdd(tctr, 1u);  // ticket after next (published after a barrier)

        // ---------------- 2.+3. gates on MFMA, gate math and local scan ----------------
        // tile 0 (rows 0..31) on MFMA first; then tile 0's gate math element j is issued
        // next to tile 1's MFMA step j, so the matrix core and the VALU work side by side
        f32x16 accB[kNT][2], accP[kNT][2];
        float psc[kNT], bsc[kNT];
        {
            const int atok = 32 * ((ln >> 2) & 1) + 4 * (ln >> 3) + (ln & 3);
            const uint16_t* ap0 = ubuf + lds_row(atok) * kRow + 32 * kh;
            const uint16_t* ap1 = ubuf + lds_row(atok + 16) * kRow + 32 * kh;
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    accB[nt][0][e] = 0.0f; accP[nt][0][e] = 0.0f; accB[nt][1][e] = 0.0f; accP[nt][1][e] = 0.0f;
                }
#pragma unroll
            for (int kk = 0; kk < C::kKSteps; ++kk) {
                const bf16x8 A = *reinterpret_cast<const bf16x8*>(ap0 + 64 * (kk >> 2) + 8 * (kk & 3));
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    accB[nt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wA[nt][kk], accB[nt][0], 0, 0, 0);
                    accP[nt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wX[nt][kk], accP[nt][0], 0, 0, 0);
                }
            }
            float4 gc[kNT];
            const uint16_t* ucol[kNT];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                psc[nt] = 1.0f;
                bsc[nt] = 0.0f;
                gc[nt] = gate_tab[cw0 + 32 * nt + ln];
                ucol[nt] = ubuf + 32 * hh * kRow + cw0 + 32 * nt + ln;
            }
            static_assert(C::kKSteps == 16 || C::kKSteps == 8, "interleave");
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j < C::kKSteps) {
                    const int kk = j;
                    const bf16x8 A = *reinterpret_cast<const bf16x8*>(ap1 + 64 * (kk >> 2) + 8 * (kk & 3));
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt) {
                        accB[nt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wA[nt][kk], accB[nt][1], 0, 0, 0);
                        accP[nt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wX[nt][kk], accP[nt][1], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    const int row = 4 * ((j >> 2) ^ (3 * hh)) + (j & 3);
                    const float u = bf2f(ucol[nt][row * kRow]);
                    const GateOut g = gate_fast(accB[nt][0][j], accP[nt][0][j], gc[nt].x, gc[nt].y, gc[nt].z, u);
                    bsc[nt] = __builtin_fmaf(g.a, bsc[nt], g.v);
                    psc[nt] = psc[nt] * g.a;
                    accB[nt][0][j] = bsc[nt];
                    accP[nt][0][j] = psc[nt];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    const int row = 16 + 4 * ((j >> 2) ^ (3 * hh)) + (j & 3);
                    const float u = bf2f(ucol[nt][row * kRow]);
                    const GateOut g = gate_fast(accB[nt][1][j], accP[nt][1][j], gc[nt].x, gc[nt].y, gc[nt].z, u);
                    bsc[nt] = __builtin_fmaf(g.a, bsc[nt], g.v);
                    psc[nt] = psc[nt] * g.a;
                    accB[nt][1][j] = bsc[nt];
                    accP[nt][1][j] = psc[nt];
                }
            }
        }
        // segment aggregates: low half-wave (tokens 0..31) then high half-wave (32..63)
        float p_lo[kNT], b_lo[kNT], A_seg[kNT], B_seg[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const float p_o = __shfl_xor(psc[nt], 32), b_o = __shfl_xor(bsc[nt], 32);
            p_lo[nt] = hh ? p_o : psc[nt];
            b_lo[nt] = hh ? b_o : bsc[nt];
            const float p_hi = hh ? psc[nt] : p_o, b_hi = hh ? bsc[nt] : b_o;
            A_seg[nt] = p_lo[nt] * p_hi;
            B_seg[nt] = __builtin_fmaf(p_hi, b_lo[nt], b_hi);
        }

        // ---------------- 4. carry: probe now, GELU while the probe is in flight ----------------
        const bool lb_lane = (kNT == 2) || (hh == 0);
        const int nt_lb = (kNT == 2) ? hh : 0;
        const size_t chl = (size_t)head * BS + cw0 + 32 * nt_lb + ln;
        const size_t wstride = (size_t)B * D;
        unsigned long long* wself = a.words + (size_t)seg * wstride + (size_t)b * D + chl;
        unsigned long long w1 = kNotReady;
        float carry_mine = 0.0f;
        if (lb_lane) {
            if (seg > 0) w1 = ld_word(wself - wstride);
            else if (a.h0 != nullptr) carry_mine = a.h0[(size_t)b * D + chl];
        }
        // y of this segment has been in LDS since the previous iteration: out_t = h_t g_t with
        // h_t = b_t + p_t c, kept as (b_t g_t, p_t g_t) until the carry c is known
        if (!last) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const uint16_t* ycol = ycur + 32 * hh * BS + cw0 + 32 * nt + ln;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float g = gelu_fast(bf2f(ycol[(16 * mt + j) * BS]));
                        accB[nt][mt][j] *= g;
                        accP[nt][mt][j] *= g;
                    }
                }
            }
        }
        if (lb_lane) {
            const float As = (kNT == 2 && hh) ? A_seg[kNT - 1] : A_seg[0];
            const float Bs = (kNT == 2 && hh) ? B_seg[kNT - 1] : B_seg[0];
            if (seg > 0) carry_mine = look_back(wself, wstride, seg, w1, As, Bs, !last, a.header);
        }
        // this wave's DMA of the next segment completes before the next iteration's barrier,
        // and before the stores below are issued (so that wait never waits for them)
        wait_vmem_all();
        if (lb_lane) {
            const float As = (kNT == 2 && hh) ? A_seg[kNT - 1] : A_seg[0];
            const float Bs = (kNT == 2 && hh) ? B_seg[kNT - 1] : B_seg[0];
            if (!last) st_word(wself, make_word(As, __builtin_fmaf(As, carry_mine, Bs), true));
            if (seg > 0) st_word(wself - wstride, kNotReady);
        }
        float state_in[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const float c = __shfl(carry_mine, ln + 32 * (kNT == 2 ? nt : 0));
            state_in[nt] = hh ? __builtin_fmaf(p_lo[nt], c, b_lo[nt]) : c;
        }
        if (cl_act)
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.conv_last) + ((size_t)b * 3 + tid / kClCh) * D +
                                      (size_t)head * BS + (tid % kClCh) * 8) = cl_rows;

        // ---------------- 5. fix-up and store ----------------
        {
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<uint16_t*>(a.out) + ((size_t)b * T + t0) * D);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const int chw = head * BS + cw0 + 32 * nt + ln;
                const int voff = (32 * hh * (int)D + chw) * 2;
                if (!last) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                        for (int j = 0; j < 16; j += 2) {
                            const float o0 = __builtin_fmaf(accP[nt][mt][j], state_in[nt], accB[nt][mt][j]);
                            const float o1 = __builtin_fmaf(accP[nt][mt][j + 1], state_in[nt], accB[nt][mt][j + 1]);
                            const uint32_t o01 = pack2bf(o0, o1);
                            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)o01, ro, voff, (16 * mt + j) * rowb, 0);
                            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(o01 >> 16), ro, voff, (16 * mt + j + 1) * rowb, 0);
                        }
                    }
                } else {
                    const uint16_t* ycol = ycur + 32 * hh * BS + cw0 + 32 * nt + ln;
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int tok = 32 * hh + 16 * mt + j;
                            const float h = __builtin_fmaf(accP[nt][mt][j], state_in[nt], accB[nt][mt][j]);
                            const float o = h * gelu_fast(bf2f(ycol[(16 * mt + j) * BS]));
                            if (tok < nt_tok)
                                __builtin_amdgcn_raw_buffer_store_b16(f2bf(o), ro, voff, (16 * mt + j) * rowb, 0);
                            if (a.h_last != nullptr && t0 + tok == T - 1) a.h_last[(size_t)b * D + chw] = h;
                        }
                    }
                }
            }
        }
        if (tid == 0) s_tk[0] = pending;
        cur = nxt;
        ++it;
    }

    wait_vmem_all();  // no DMA into LDS may outlive the workgroup
    if (tid0 == 0) {
        const unsigned done = atomicAdd(&a.header[kDoneWord], 1u);
        if (done == G - 1) {
            for (int h = 0; h < a.H; ++h) atomicExch(&a.header[kTicketWord + h], 0u);
            atomicExch(&a.header[kDoneWord], 0u);
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

// Compute units of the current device (cached per device).
static int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

hipError_t launch_prefill(const PrefillArgs& a_in, int dtype, int bs, hipStream_t s) {
    PrefillArgs a = a_in;
    if (dtype == 1) {
        // persistent: one workgroup per CU, the same number for every head
        const int ncu = device_cu_count();
        a.wph = ncu > a.H ? ncu / a.H : 1;
        const dim3 grid(a.wph * a.H);
        if (bs == 256)
            hipLaunchKernelGGL((prefill_bf16_kernel<256>), grid, dim3(PCfg<256>::kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((prefill_bf16_kernel<128>), grid, dim3(PCfg<128>::kThreads), 0, s, a);
    } else {
        const dim3 grid(a.n_units);
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
