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
#include <algorithm>
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
    // the stride goes through an opaque SGPR copy: the window offsets are then formed here with
    // scalar ops, not hoisted out of the caller's loop (where they would be spilled to VGPR lanes)
    asm volatile("" : "+s"(wstride));
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
        const float ikc = gate_ikc(sp);        // log2(a) = kc * r, ikc = 1 / kc
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
                const GateOut g = kBf ? gate_fast(accB[mt][j], accP[mt][j], nba, nbx, ikc, u)
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
}

// ---------------------------------------------------------------------------------------
// bf16 storage, persistent kernel (the measured path).
//
// One workgroup per CU, pinned to one gate head for its lifetime: wave w keeps the MFMA B
// fragments of output channels [32w, 32w+32) of both gate blocks in VGPRs (128 registers), so
// the gate weights are read once per workgroup.  The workgroup walks the head's segments in
// ticket order (segment-major over the batch), one segment ahead in the conv:
//   iteration k: [MFMA tile 0 of segment k  | conv of segment k+1 -> u[(k+1)&1]]
//                copies: x of segment k+2, y of segment k
//                [MFMA tile 1 of segment k  | gate math + scan of tile 0] [gate math tile 1]
//                wait for the copies; [carry probe | GELU merge] [look-back, publish]
//                [fix-up -> LDS -> 16-byte stores] barrier
// Every wave copies (global -> LDS, no VGPRs) exactly the x rows its conv lanes read and the y
// rows its output lanes read, into regions of its own, so readiness is a wave-local wait and
// the barrier only orders u (written by all waves, double-buffered).  Rows before token 0
// come from the carried conv window (or a zero block) by the same copies.
// Placement: the hardware deals workgroups to the 8 XCDs round-robin; consecutive slots of
// one XCD are given to one head, so each XCD's L2 serves few heads.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffff, 0x00020000);
}

__device__ __forceinline__ float dot2bf(uint32_t w, uint32_t x, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, x), c, false);
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xc07f); }   // lgkmcnt(0)

// Workgroup barrier that orders LDS accesses only.  __syncthreads() would also wait for every
// outstanding global->LDS copy (its fence must cover their LDS writes); here each wave waits for
// its own copies where it reads them, so the barrier only needs this wave's LDS accesses done.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int BS>
struct PCfg {
    static constexpr int kWaves = BS / 32;          // wave w: output channels 32w .. 32w+31
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kRow = BS + 8;             // u row stride (bf16 elements)
    static constexpr int kKSteps = BS / 16;
    // conv tile of a wave: 64 channel pairs (128 channels) x 16 tokens
    static constexpr int kPairWaves = BS / 128;     // waves per token group
    static constexpr int kTokGroups = kWaves / kPairWaves;
    static constexpr int kTok = kSeg / kTokGroups;
    static constexpr int kXRows = 20;               // tokens 16 tg - 3 .. 16 tg + 16 (one spare)
    static constexpr int kXElems = kXRows * 128;
    // y / output staging region of a wave: 64 rows x 32 channels; rows 32..63 start 64 bytes
    // later so that the two half-waves' 2-byte accesses fall in different banks
    static constexpr int kYElems = kSeg * 32 + 32;
    static_assert(kTok == 16 && kKSteps * 16 == BS, "tiling");
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int yrow(int r) { return r * 32 + ((r >> 5) << 5); }

// Global -> LDS copies of one wave (buffer loads with the LDS bit: SGPR base, 32-bit lane
// offsets, no VGPR data).  x: rows t0 + 16 tg - 3 + r (r = 0..19) of the wave's 128 channels
// (16 lanes per 256-byte row, 4 rows per instruction); rows past T-1 repeat row T-1 (never
// used); for segment 0 the rows before token 0 come from the conv window, read through a
// resource of length 0 when there is none (out-of-range buffer reads return zeros).  A ticket
// past the end copies the last ticket's rows again (harmless, never used).
__device__ __forceinline__ void dma_x_rows(const PrefillArgs& a, int head, int bs, int pw, int tg,
                                           unsigned tk, unsigned n_tk, int lane, uint16_t* dst) {
    tk = min(tk, n_tk - 1);
    const int seg = (int)(tk / (unsigned)a.B), b = (int)(tk % (unsigned)a.B);
    const int rowb = a.D * 2;
    const int coff = (head * bs + 128 * pw + 8 * (lane & 15)) * 2;
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(static_cast<const uint16_t*>(a.x) + (size_t)b * a.T * a.D);
    const int tok0 = seg * kSeg + 16 * tg - 3 + (lane >> 4);
    if (seg == 0 && tg == 0) {
        // rows 0..2 of the first instruction are tokens -3..-1 (the resource is formed before the
        // lane-divergent choice, from a pointer made visibly wave-uniform)
        // (readfirstlane yields a signed int: both halves are widened as unsigned)
        const uint64_t cp = reinterpret_cast<uint64_t>(a.conv0 ? a.conv0 : a.x);
        const uint32_t c_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(cp >> 32));
        const uint32_t c_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)cp);
        const uint64_t cpu = ((uint64_t)c_hi << 32) | (uint64_t)c_lo;
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void*>(cpu), 0, a.conv0 ? 0xffffffffu : 0u, 0x00020000);
        const bool from_x = (lane >> 4) == 3;
        if (from_x) __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, dst, 16, coff, 0, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, dst, 16, (((b * 3 + (lane >> 4)) * a.D) * 2) + coff, 0, 0, 0);
    } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, dst, 16, min(tok0, a.T - 1) * rowb + coff, 0, 0, 0);
    }
#pragma unroll
    for (int q = 1; q < 5; ++q) {
        const int tok = min(tok0 + 4 * q, a.T - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, dst + q * 512, 16, tok * rowb + coff, 0, 0, 0);
    }
}

// y: rows t0 .. t0+63 (clamped to T-1) of the wave's 32 channels (4 lanes per 64-byte row).
__device__ __forceinline__ void dma_y_rows(const PrefillArgs& a, int head, int bs, int cw0,
                                           unsigned tk, unsigned n_tk, int lane, uint16_t* dst) {
    tk = min(tk, n_tk - 1);
    const int seg = (int)(tk / (unsigned)a.B), b = (int)(tk % (unsigned)a.B);
    const int rowb = a.D * 2;
    const int coff = (head * bs + cw0 + 8 * (lane & 3)) * 2;
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(static_cast<const uint16_t*>(a.y) + (size_t)b * a.T * a.D);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int tok = min(seg * kSeg + 16 * q + (lane >> 2), a.T - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, dst + yrow(16 * q), 16, tok * rowb + coff, 0, 0, 0);
    }
}

// A copy of v that the compiler cannot see through: values derived from it inside the loop
// are recomputed there instead of being kept live across it (the gate weights already occupy
// half of the register file).
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// The same for a wave-uniform value (kept in an SGPR).
__device__ __forceinline__ int sopaque(int v) {
    asm volatile("" : "+s"(v));
    return v;
}

template <int BS>
__global__ void __launch_bounds__(PCfg<BS>::kThreads)
prefill_bf16_kernel(PrefillArgs a) {
    using C = PCfg<BS>;
    constexpr int kRow = C::kRow;
    constexpr int kU = kSeg * kRow;  // elements of one u tile
    // LDS.  In the loop every access is "flat array + one index formed once per iteration
    // (opaque to the optimizer) + constants": the compiler then knows which array each access
    // touches, and an LDS read never waits for a global->LDS copy into another array.  (Left to
    // itself it splits addresses into long pointer chains and loses that knowledge, and then
    // every LDS read waits for all copies in flight.)
    __shared__ __attribute__((aligned(16))) uint16_t u_lds[2 * kU];                    // u tiles
    __shared__ __attribute__((aligned(16))) uint16_t x_lds[C::kWaves * C::kXElems];    // x rows
    __shared__ __attribute__((aligned(16))) uint16_t y_lds[C::kWaves * C::kYElems];    // y rows / out
    __shared__ __attribute__((aligned(16))) uint4 conv_tab[BS / 2];   // taps of a channel pair
    __shared__ __attribute__((aligned(8))) float2 convb_tab[BS / 2];  // biases of a channel pair
    __shared__ __attribute__((aligned(16))) float4 gate_tab[BS];      // (nba, nbx, 1/kc, 0) per channel
    __shared__ unsigned s_tk[4];
    const uint32_t* const x_lds32 = reinterpret_cast<const uint32_t*>(x_lds);
    uint32_t* const u_lds32 = reinterpret_cast<uint32_t*>(u_lds);

    const int tid0 = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int B = a.B, T = a.T;
    const size_t D = (size_t)a.D;
    const int rowb = (int)(D * 2);

    // ---- placement: slot -> head ----
    const unsigned G = gridDim.x, bid = blockIdx.x;
    const unsigned xcd = bid & 7u, jx = bid >> 3, per = G >> 3, rem = G & 7u;
    const unsigned slot = xcd * per + min(xcd, rem) + jx;
    const int head_ = (int)(slot / (unsigned)a.wph);
    unsigned* tctr = a.header + kTicketWord + head_;
    const unsigned n_tk = (unsigned)(B * a.S);

    const int pw = wv % C::kPairWaves, tg = wv / C::kPairWaves;  // conv tile
    const int cw0_ = 32 * wv;                                      // output channels
    const int xw0_ = wv * C::kXElems, yw0_ = wv * C::kYElems;      // the wave's LDS regions
    const int head = head_, cw0 = cw0_, xw0 = xw0_, yw0 = yw0_;
    // conv rows of this wave's tokens 16 tg + k: lds_row(16 tg + k) = 16 tg + (k ^ 12 sw)
    const int csw = 12 * ((tg >> 1) & 1);

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
        gate_tab[i] = make_float4(-bia * kLog2e, -bix * kLog2e, gate_ikc(sp), 0.0f);
    }
    // gate weights of this wave's channels, held in registers throughout
    bf16x8 wA[C::kKSteps], wX[C::kKSteps];
    {
        const int lane = tid0 & 63, ln = lane & 31, kh = lane >> 5;
        const size_t chn = (size_t)head * BS + cw0 + ln;
        const uint16_t* war = static_cast<const uint16_t*>(a.wa) + chn * BS;
        const uint16_t* wxr = static_cast<const uint16_t*>(a.wx) + chn * BS;
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk) {
            // K order: lane half kh supplies elements [64 q + 32 kh + 8 s, +8) at step 4q + s
            const int kb = 64 * (kk >> 2) + 32 * kh + 8 * (kk & 3);
            wA[kk] = *reinterpret_cast<const bf16x8*>(war + kb);
            wX[kk] = *reinterpret_cast<const bf16x8*>(wxr + kb);
        }
    }

    // ---- prologue: tickets for this workgroup's first three segments; conv of the first ----
    if (tid0 == 0) s_tk[0] = atomicAdd(tctr, 1u);
    __syncthreads();  // tables and the first ticket
    // tickets are workgroup-uniform: kept in SGPRs (buffer resources are built from them)
    unsigned cur = __builtin_amdgcn_readfirstlane(s_tk[0]);
    unsigned n1, n2;
    {
        const int lane = tid0 & 63;
        dma_x_rows(a, head, BS, pw, tg, cur, n_tk, lane, x_lds + xw0);
        wait_vmem_all();
        const int cp = 64 * pw + lane;
        const uint4 wq = conv_tab[cp];
        const float2 cb = convb_tab[cp];
#pragma unroll
        for (int k = 0; k < C::kTok; ++k) {
            const uint32_t* xw = x_lds32 + xw0 / 2 + lane;
            const uint32_t x0 = xw[k * 64], x1 = xw[(k + 1) * 64], x2 = xw[(k + 2) * 64], x3 = xw[(k + 3) * 64];
            const float u0 = dot2bf(wq.y, __builtin_amdgcn_perm(x3, x2, 0x05040100u),
                                    dot2bf(wq.x, __builtin_amdgcn_perm(x1, x0, 0x05040100u), cb.x));
            const float u1 = dot2bf(wq.w, __builtin_amdgcn_perm(x3, x2, 0x07060302u),
                                    dot2bf(wq.z, __builtin_amdgcn_perm(x1, x0, 0x07060302u), cb.y));
            u_lds32[(lds_row(tg * C::kTok + k) * kRow) / 2 + cp] = pack2bf(u0, u1);
        }
        // The next two tickets are taken only now, a conv after the first: by then every
        // workgroup of the head has normally taken its first ticket, so a head with few
        // segments spreads them over all its workgroups instead of three each to the first
        // workgroups to arrive.  (No copy into LDS is in flight here.)
        if (tid0 == 0) {
            s_tk[1] = atomicAdd(tctr, 1u);
            s_tk[2] = atomicAdd(tctr, 1u);
        }
        lds_barrier();  // the two tickets are visible; this wave's conv reads of x are complete
        n1 = __builtin_amdgcn_readfirstlane(s_tk[1]);
        n2 = __builtin_amdgcn_readfirstlane(s_tk[2]);
        dma_x_rows(a, head, BS, pw, tg, n1, n_tk, lane, x_lds + xw0);
    }
    unsigned pending = 0;  // taken once per iteration, published at the iteration's barrier
    wait_vmem_all();
    lds_barrier();  // u of the first segment complete; every wave has read the ticket slots
    unsigned it = 0;

    while (cur < n_tk) {
        // per-iteration copies of workgroup constants: values derived from them are formed
        // here with scalar ops instead of being hoisted (and spilled) across the loop
        const int xw0 = sopaque(xw0_), yw0 = sopaque(yw0_), cw0 = sopaque(cw0_), head = sopaque(head_);
        const int tid = opaque(tid0);
        const int lane = tid & 63, ln = lane & 31, kh = lane >> 5, hh = lane >> 5;
        const int seg = (int)(cur / (unsigned)B), b = (int)(cur % (unsigned)B);
        const int t0 = seg * kSeg;
        const int nt_tok = min(kSeg, T - t0);
        const bool last = (seg == a.S - 1);
        const int ucur = sopaque((int)(it & 1) * kU), unxt = kU - ucur;  // u tiles of cur, n1
        const int atok = 32 * ((ln >> 2) & 1) + 4 * (ln >> 3) + (ln & 3);

        // ------- 1. MFMA tile 0 (tokens 0..31) of `cur`, interleaved with the conv of `n1` -------
        f32x16 accB[2], accP[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            accB[0][e] = 0.0f; accP[0][e] = 0.0f; accB[1][e] = 0.0f; accP[1][e] = 0.0f;
        }
        {
            const int cp = 64 * pw + lane;
            const uint4 wq = conv_tab[cp];
            const float2 cb = convb_tab[cp];
            const int ia0 = opaque(ucur + lds_row(atok) * kRow + 32 * kh);
            const int ixr = opaque(xw0 / 2 + lane);
            const int iuw = opaque((unxt + 16 * tg * kRow) / 2 + cp);
            uint32_t xr[C::kTok + 3];
#pragma unroll
            for (int k = 0; k < C::kTok + 3; ++k) xr[k] = x_lds32[ixr + k * 64];
            constexpr int kTokPerStep = C::kTok / C::kKSteps;  // conv tokens per MFMA k-step
            // the row swizzle of this wave's tokens is a compile-time constant in each branch,
            // so every u store has an immediate offset
            auto tile0 = [&](auto sw) {
                constexpr int kSw = decltype(sw)::value;
#pragma unroll
                for (int kk = 0; kk < C::kKSteps; ++kk) {
                    const bf16x8 A = *reinterpret_cast<const bf16x8*>(u_lds + ia0 + 64 * (kk >> 2) + 8 * (kk & 3));
                    accB[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wA[kk], accB[0], 0, 0, 0);
                    accP[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wX[kk], accP[0], 0, 0, 0);
#pragma unroll
                    for (int s2 = 0; s2 < kTokPerStep; ++s2) {
                        const int k = kk * kTokPerStep + s2;
                        // (x_{t-3}, x_{t-2}) and (x_{t-1}, x_t) of each of the two channels
                        const uint32_t p0a = __builtin_amdgcn_perm(xr[k + 1], xr[k], 0x05040100u);
                        const uint32_t p0b = __builtin_amdgcn_perm(xr[k + 1], xr[k], 0x07060302u);
                        const uint32_t p2a = __builtin_amdgcn_perm(xr[k + 3], xr[k + 2], 0x05040100u);
                        const uint32_t p2b = __builtin_amdgcn_perm(xr[k + 3], xr[k + 2], 0x07060302u);
                        const float u0 = dot2bf(wq.y, p2a, dot2bf(wq.x, p0a, cb.x));
                        const float u1 = dot2bf(wq.w, p2b, dot2bf(wq.z, p0b, cb.y));
                        u_lds32[iuw + ((k ^ kSw) * kRow) / 2] = pack2bf(u0, u1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if (sopaque(csw) != 0) tile0(std::integral_constant<int, 12>{});
            else tile0(std::integral_constant<int, 0>{});
        }
        // Copies go out only here, after this iteration's last LDS store before the wait in
        // step 4 (an LDS store issued while a global->LDS copy is in flight waits for the copy):
        // the x rows of the segment after next (the conv's reads are complete) and this
        // segment's y rows (the region's previous contents were stored out last iteration).
        wait_lds_all();
        dma_x_rows(a, head, BS, pw, tg, n2, n_tk, lane, x_lds + xw0);
        dma_y_rows(a, head, BS, cw0, cur, n_tk, lane, y_lds + yw0);

        // ------- 2.+3. tile 1 on MFMA next to tile 0's gate math; then tile 1's gate math -------
        float psc = 1.0f, bsc = 0.0f;
        {
            const int ia1 = opaque(ucur + lds_row(atok + 16) * kRow + 32 * kh);
            const float4 gc = gate_tab[cw0 + ln];
            // u of (token 32 hh + 16 mt + j, channel cw0 + ln) is at row 32 hh + 16 mt + (j ^ 12 hh);
            // with j = 4 g + m that is 32 hh + 16 mt + 4 g + m + hh (12 - 8 g): one base per g
            int iub[4];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) iub[g4] = opaque(ucur + (32 * hh + hh * (12 - 8 * g4)) * kRow + cw0 + ln);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j < C::kKSteps) {
                    const bf16x8 A = *reinterpret_cast<const bf16x8*>(u_lds + ia1 + 64 * (j >> 2) + 8 * (j & 3));
                    accB[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wA[j], accB[1], 0, 0, 0);
                    accP[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wX[j], accP[1], 0, 0, 0);
                }
                const float u = bf2f(u_lds[iub[j >> 2] + j * kRow]);
                const GateOut g = gate_fast(accB[0][j], accP[0][j], gc.x, gc.y, gc.z, u);
                bsc = __builtin_fmaf(g.a, bsc, g.v);
                psc = psc * g.a;
                accB[0][j] = bsc;
                accP[0][j] = psc;
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float u = bf2f(u_lds[iub[j >> 2] + (16 + j) * kRow]);
                const GateOut g = gate_fast(accB[1][j], accP[1][j], gc.x, gc.y, gc.z, u);
                bsc = __builtin_fmaf(g.a, bsc, g.v);
                psc = psc * g.a;
                accB[1][j] = bsc;
                accP[1][j] = psc;
            }
        }
        // segment aggregate: low half-wave (tokens 0..31) then high half-wave (32..63)
        const float p_o = __shfl_xor(psc, 32), b_o = __shfl_xor(bsc, 32);
        const float p_lo = hh ? p_o : psc, b_lo = hh ? b_o : bsc;
        const float p_hi = hh ? psc : p_o, b_hi = hh ? bsc : b_o;
        const float A_seg = p_lo * p_hi;
        const float B_seg = __builtin_fmaf(p_hi, b_lo, b_hi);
        const size_t chl = (size_t)head * BS + cw0 + ln;
        const size_t wstride = (size_t)B * D;
        unsigned long long* const wself = a.words + (size_t)seg * wstride + (size_t)b * D + chl;
        unsigned long long* const wprev = wself - wstride;

        // ------- 4. carry: y and the next x have landed; probe, then GELU while it is in flight -------
        if (tid == 0) pending = atomicAdd(tctr, 1u);  // ticket three segments ahead
        wait_vmem_all();
        // the aggregate goes out now (after the wait, so that wait never includes this store):
        // successors can fold it while this workgroup merges the GELU branch and looks back
        if (hh == 0 && seg > 0 && !last) st_word(wself, make_word(A_seg, B_seg, false));
        unsigned long long w1 = kNotReady;
        float h0v = 0.0f;
        if (hh == 0) {
            if (seg > 0) w1 = ld_word(wprev);
            else if (a.h0 != nullptr) h0v = a.h0[(size_t)b * D + chl];
        }
        // out_t = h_t g_t with h_t = b_t + p_t c: kept as (b_t g_t, p_t g_t) until c is known
        const int iy = opaque(yw0 + yrow(32 * hh) + ln);  // y / staging of (token 32 hh + r, this lane)
        if (!last) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float g = gelu_fast(bf2f(y_lds[iy + (16 * mt + j) * 32]));
                    accB[mt][j] *= g;
                    accP[mt][j] *= g;
                }
            }
        }
        float carry = h0v;
        if (hh == 0 && seg > 0) carry = look_back(wself, wstride, seg, w1, A_seg, B_seg, false, a.header);
        wait_vmem_all();  // the carry's loads (nothing else is outstanding): no wait after the stores
        const unsigned long long winc = make_word(A_seg, __builtin_fmaf(A_seg, carry, B_seg), true);
        if (hh == 0 && !last) st_word(wself, winc);
        carry = __shfl(carry, ln);
        const float state_in = hh ? __builtin_fmaf(p_lo, carry, b_lo) : carry;

        // ------- 5. fix-up into the wave's staging region (in place of y), then 16-byte stores -------
        if (!last) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    const float o0 = __builtin_fmaf(accP[mt][j], state_in, accB[mt][j]);
                    const float o1 = __builtin_fmaf(accP[mt][j + 1], state_in, accB[mt][j + 1]);
                    // opaque: otherwise the compiler converts o1 a second time for the high half
                    // instead of storing that half with ds_write_b16_d16_hi
                    const uint32_t o01 = (uint32_t)opaque((int)pack2bf(o0, o1));
                    y_lds[iy + (16 * mt + j) * 32] = (uint16_t)o01;
                    y_lds[iy + (16 * mt + j + 1) * 32] = (uint16_t)(o01 >> 16);
                }
            }
        } else {
            // last segment: GELU here, h_last and the conv window after the last token
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int tok = 32 * hh + 16 * mt + j;
                    const float h = __builtin_fmaf(accP[mt][j], state_in, accB[mt][j]);
                    const float o = h * gelu_fast(bf2f(y_lds[iy + (16 * mt + j) * 32]));
                    y_lds[iy + (16 * mt + j) * 32] = f2bf(o);
                    if (a.h_last != nullptr && t0 + tok == T - 1) a.h_last[(size_t)b * D + chl] = h;
                }
            }
            if (a.conv_last != nullptr && tg == 0 && lane < 48) {
                // the last three inputs (oldest first); before token 0 they are the carried window
                // (read here, after the carry wait, so an in-place window was read by segment 0 first)
                const int rr = lane >> 4, tok = T - 3 + rr;
                const size_t c = (size_t)head * BS + 128 * pw + 8 * (lane & 15);
                uint4 v = make_uint4(0, 0, 0, 0);
                if (tok >= 0)
                    v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + ((size_t)b * T + tok) * D + c);
                else if (a.conv0 != nullptr)
                    v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.conv0) + ((size_t)b * 3 + 3 + tok) * D + c);
                *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.conv_last) + ((size_t)b * 3 + rr) * D + c) = v;
            }
        }
        {
            // rows of the staging region -> out (4 lanes per 64-byte row, 16 rows per step)
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<uint16_t*>(a.out) + ((size_t)b * T + t0) * D);
            const int voff = (int)((size_t)head * BS + cw0 + 8 * (lane & 3)) * 2;
            const int iyr = opaque(yw0 + (lane >> 2) * 32 + 8 * (lane & 3));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 16 * q + (lane >> 2);
                const uint4 v = *reinterpret_cast<const uint4*>(y_lds + iyr + yrow(16 * q));
                if (r < nt_tok)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, voff + r * rowb, 0, 0);
            }
        }
        if (tid == 0) s_tk[it & 3] = pending;
        lds_barrier();  // u of n1 complete and u of cur no longer read; the ticket slot is visible
        const unsigned n3 = __builtin_amdgcn_readfirstlane(s_tk[it & 3]);
        cur = n1;
        n1 = n2;
        n2 = n3;
        ++it;
    }

    wait_vmem_all();  // no copy into LDS may outlive the workgroup
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

// The look-back state of one call, set up on the stream before the scan kernel: the header
// (error flags, ticket counters, zero block) cleared, and every carry word the call can read
// (segments 0 .. S-2; the last segment publishes none) set to "not ready" with 16-byte stores.
// Whatever the buffer held before (a fresh allocation, another shape's words, a call that
// stopped at a spin limit) is overwritten, so no call depends on an earlier one.
__global__ void __launch_bounds__(256) ws_reset_kernel(unsigned* header, uint4* words, size_t n16) {
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < (int)(kWsHeader / 4); i += 256) header[i] = 0u;
    }
    const uint4 nr = make_uint4(~0u, ~0u, ~0u, ~0u);
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) words[i] = nr;
}

hipError_t launch_ws_reset(const PrefillArgs& a, hipStream_t s) {
    // words of segments 0 .. S-2, two per 16-byte store (B * D is even: D % 8 == 0)
    const size_t n16 = (size_t)(a.S - 1) * (size_t)a.B * (size_t)a.D / 2;
    const size_t blocks = std::min<size_t>(std::max<size_t>((n16 + 1023) / 1024, 1), 4096);
    hipLaunchKernelGGL(ws_reset_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.header,
                       reinterpret_cast<uint4*>(a.words), n16);
    return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cu_count() {
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
    const hipError_t er = launch_ws_reset(a, s);
    if (er != hipSuccess) return er;
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
