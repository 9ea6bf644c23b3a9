// Device helpers shared by the RG-LRU kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rglru {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef float f32x16 __attribute__((__vector_size__(64)));
typedef float f32x4 __attribute__((__vector_size__(16)));

constexpr float kLog2e = 1.4426950408889634f;
// GELU, tanh form (Hendrycks & Gimpel 2016): gelu(y) = 0.5 y (1 + tanh(k (y + 0.044715 y^3)))
// with k = sqrt(2/pi).  Since 0.5 (1 + tanh(z)) = 1 / (1 + exp(-2z)), the fast form is
// y / (1 + 2^(y (G1 + G2 y^2))) with G1 = -2 k log2(e), G2 = 0.044715 G1.
constexpr float kGeluK = 0.7978845608028654f;
constexpr float kGeluG1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
constexpr float kGeluG2 = 0.044715f * kGeluG1;

// ---------------------------------------------------------------------------------------
// storage types: fp32 (float) or bf16 (uint16_t bits)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// round-to-nearest-even (hardware v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

template <typename ST> struct Store;

template <> struct Store<float> {
    static constexpr bool kBf16 = false;
    __device__ static __forceinline__ float get(const float* p, size_t i) { return p[i]; }
    __device__ static __forceinline__ void put(float* p, size_t i, float v) { p[i] = v; }
    // 8 consecutive elements (32 bytes) -> fp32
    __device__ static __forceinline__ void load8(const float* p, float (&v)[8]) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    __device__ static __forceinline__ void store8(float* p, const float (&v)[8]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
};

template <> struct Store<uint16_t> {
    static constexpr bool kBf16 = true;
    __device__ static __forceinline__ float get(const uint16_t* p, size_t i) { return bf2f(p[i]); }
    __device__ static __forceinline__ void put(uint16_t* p, size_t i, float v) { p[i] = f2bf(v); }
    __device__ static __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
        v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
    }
    __device__ static __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
        *reinterpret_cast<uint4*>(p) = make_uint4(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]),
                                                  pack2bf(v[4], v[5]), pack2bf(v[6], v[7]));
    }
};

// ---------------------------------------------------------------------------------------
// per-channel gate constants
// ---------------------------------------------------------------------------------------
// softplus(-L) = -log(sigmoid(L)) = max(-L, 0) + log1p(exp(-|L|)): no cancellation for
// either sign of L, and no branch.
__device__ __forceinline__ float softplus_neg(float lam) {
    return fmaxf(-lam, 0.0f) + log1pf(expf(-fabsf(lam)));
}

// 1 / kc for gate_fast, kc = -8 softplus(-Lambda) log2(e) <= 0; kc = -0 (a == 1 for every r)
// maps to -FLT_MAX, which keeps (1 + er) * ikc free of 0 * inf.
__device__ __forceinline__ float gate_ikc(float sp_neg) {
    return fmaxf(1.0f / (-8.0f * sp_neg * kLog2e), -3.4028234663852886e38f);
}

// ---------------------------------------------------------------------------------------
// RG-LRU gate arithmetic for one element (r, i, a and the gated input v = sqrt(1-a^2) i u)
//
// Fast form (bf16 storage): exp2/rcp/sqrt hardware approximations (about 1 ulp each).
//   pre-activations arrive as MFMA sums without bias; nb = -bias * log2(e);
//   kc = -8 softplus(-Lambda) log2(e) (so log2(a) = kc * r) enters as ikc = 1 / kc: then
//   kc * r = kc / (1 + er) = rcp((1 + er) * ikc), one reciprocal and no multiply.
// Precise form (fp32 storage): library expf/expm1f and IEEE division; sqrt(1 - a^2) is
//   computed as sqrt(-expm1(2 log a)) so it keeps full relative accuracy when a -> 1.
// ---------------------------------------------------------------------------------------
struct GateOut {
    float a, v;
};

__device__ __forceinline__ GateOut gate_fast(float sa, float sx, float nba, float nbx, float ikc,
                                             float u) {
    const float er = __builtin_amdgcn_exp2f(__builtin_fmaf(sa, -kLog2e, nba));
    const float ei = __builtin_amdgcn_exp2f(__builtin_fmaf(sx, -kLog2e, nbx));
    const float i = __builtin_amdgcn_rcpf(1.0f + ei);
    // r -> 0 (er -> inf) gives rcp(-inf) = -0 and a = 1
    const float a = __builtin_amdgcn_exp2f(__builtin_amdgcn_rcpf(__builtin_fmaf(er, ikc, ikc)));
    // a <= 1 in exact arithmetic; when the 1-ulp error of the hardware exp2 puts a just above
    // 1, 1 - a^2 is a rounding-sized negative number and |1 - a^2| is as good an estimate of
    // the true (tiny, non-negative) value as 0.  The absolute value is a free operand modifier.
    const float m = __builtin_amdgcn_sqrtf(fabsf(__builtin_fmaf(-a, a, 1.0f)));
    return {a, m * (i * u)};
}

// ba, bx: biases; kcn = -8 softplus(-Lambda) (natural-log units).
__device__ __forceinline__ GateOut gate_precise(float sa, float sx, float ba, float bx, float kcn,
                                                float u) {
    const float r = 1.0f / (1.0f + expf(-(sa + ba)));
    const float i = 1.0f / (1.0f + expf(-(sx + bx)));
    const float la = kcn * r;
    const float a = expf(la);
    const float m = sqrtf(-expm1f(2.0f * la));
    return {a, m * (i * u)};
}

__device__ __forceinline__ float gelu_fast(float y) {
    const float z = y * __builtin_fmaf(kGeluG2, y * y, kGeluG1);
    return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

__device__ __forceinline__ float gelu_precise(float y) {
    return 0.5f * y * (1.0f + tanhf(kGeluK * (y + 0.044715f * y * y * y)));
}

// ---------------------------------------------------------------------------------------
// MFMA 32x32 tile layout (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2_f32), one wave:
//   operand A (M x K): lane l supplies row (l % 32), K-slice (l / 32)
//   operand B (K x N): lane l supplies column (l % 32), K-slice (l / 32)
//   result  D (32x32 fp32, 16 registers): lane l holds column (l % 32); register j holds
//   row 8*(j/4) + 4*(l/32) + (j%4).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int mfma_d_row(int lane, int j) {
    return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

}  // namespace rglru
