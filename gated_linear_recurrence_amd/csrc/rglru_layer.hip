// The residual layer's elementwise parts, for gfx950 (CDNA4).  The page "Gemma 詳解：
// RecurrentGemma 架構" (module printout, sections "含遞迴區塊的殘差區塊" and "含區域 MQA 的殘差
// 區塊") wraps each temporal-mixing block in a pre-norm residual layer:
//
//   h   = x + temporal(RMSNorm_1(x))
//   out = h + down_proj(gelu_tanh(gate_proj(RMSNorm_2(h))) * up_proj(RMSNorm_2(h)))
//
// with RMSNorm(v) = v / sqrt(mean(v^2) + eps) * g.  The projections are the bf16 MFMA GEMM of
// rglru_proj.hip (gate_proj and up_proj as one launch with two output segments).  Here:
//   add_rmsnorm_kernel  one wave per row: h = x (+ y), rounded to bf16, and RMSNorm(h) * g, from
//                       the rounded h, in fp32; either output may be skipped.  It serves both
//                       norms, the second fused with the first residual addition, and, without
//                       the norm, the final residual addition;
//   geglu_kernel        a = gelu_tanh(gate) * up, eight elements per thread, in place over gate.
#include "rglru_device.h"
#include "rglru_internal.h"

namespace rglru {
namespace {

constexpr int kNormMaxChunks = 16;   // 8-element chunks per lane: rows of up to 8192

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__global__ void __launch_bounds__(256) add_rmsnorm_kernel(NormArgs a) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.M) return;
    const int nch = a.D / 8;
    const size_t base = (size_t)row * a.D;
    const uint4* x = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + base);
    const uint4* y = a.y ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.y) + base)
                         : nullptr;
    uint4 hv[kNormMaxChunks];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kNormMaxChunks; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            uint4 v = x[c];
            if (y) {
                const uint4 w = y[c];
                v.x = pack2bf(bf_lo(v.x) + bf_lo(w.x), bf_hi(v.x) + bf_hi(w.x));
                v.y = pack2bf(bf_lo(v.y) + bf_lo(w.y), bf_hi(v.y) + bf_hi(w.y));
                v.z = pack2bf(bf_lo(v.z) + bf_lo(w.z), bf_hi(v.z) + bf_hi(w.z));
                v.w = pack2bf(bf_lo(v.w) + bf_lo(w.w), bf_hi(v.w) + bf_hi(w.w));
            }
            hv[i] = v;
            const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float lo = bf_lo(e[k]), hi = bf_hi(e[k]);
                ss = __builtin_fmaf(lo, lo, ss);
                ss = __builtin_fmaf(hi, hi, ss);
            }
            if (a.h) reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.h) + base)[c] = v;
        }
    }
    if (!a.n) return;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)a.D + a.eps);
    const uint4* g = static_cast<const uint4*>(a.g);
    uint4* n = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.n) + base);
#pragma unroll
    for (int i = 0; i < kNormMaxChunks; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            const uint4 v = hv[i], s = g[c];
            uint4 o;
            o.x = pack2bf(bf_lo(v.x) * inv * bf_lo(s.x), bf_hi(v.x) * inv * bf_hi(s.x));
            o.y = pack2bf(bf_lo(v.y) * inv * bf_lo(s.y), bf_hi(v.y) * inv * bf_hi(s.y));
            o.z = pack2bf(bf_lo(v.z) * inv * bf_lo(s.z), bf_hi(v.z) * inv * bf_hi(s.z));
            o.w = pack2bf(bf_lo(v.w) * inv * bf_lo(s.w), bf_hi(v.w) * inv * bf_hi(s.w));
            n[c] = o;
        }
    }
}

__device__ __forceinline__ uint32_t geglu2(uint32_t g, uint32_t u) {
    return pack2bf(gelu_fast(bf_lo(g)) * bf_lo(u), gelu_fast(bf_hi(g)) * bf_hi(u));
}

__global__ void __launch_bounds__(256) geglu_kernel(uint4* gate, const uint4* up, size_t n8) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const uint4 g = gate[i], u = up[i];
    gate[i] = make_uint4(geglu2(g.x, u.x), geglu2(g.y, u.y), geglu2(g.z, u.z), geglu2(g.w, u.w));
}

}  // namespace

hipError_t launch_add_rmsnorm(const NormArgs& a, hipStream_t s) {
    if (a.M == 0) return hipSuccess;
    hipLaunchKernelGGL(add_rmsnorm_kernel, dim3((unsigned)((a.M + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_geglu(void* gate, const void* up, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t n8 = n / 8;
    hipLaunchKernelGGL(geglu_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       static_cast<uint4*>(gate), static_cast<const uint4*>(up), n8);
    return hipGetLastError();
}

}  // namespace rglru
