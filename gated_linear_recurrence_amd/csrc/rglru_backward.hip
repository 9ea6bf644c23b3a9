// Backward pass of the recurrent block's temporal-mixing path, for gfx950 (CDNA4).  The pages
// give no training detail; these are the chain-rule gradients of the forward definition
// (conv k=4 -> block-diagonal gates -> RG-LRU -> times GELU-tanh of y) for
//   L = sum_t dout_t . out_t + dh_last . h_{T-1}.
//
// Intermediates are head-major, [H][B*T][256] (channel k of head h of token m at
// (h * M + m) * 256 + k), so that the three block-diagonal products are plain GEMMs of the
// projection kernel, one launch per head:
//   gates:      [Rpre | Ipre]_h = U_h [W_a[h]; W_x[h]]^T + b           (K = 256, two segments)
//   input grad: dU_h = [dRpre | dIpre]_h [W_a[h]^T | W_x[h]^T]^T       (K = 512)
//   weights:    [dW_a; dW_x]_h = [dRpre | dIpre]_h^T U_h                (K = B*T, split K, fp32)
// The scans run per channel over chunks of 64 tokens: local aggregates, a sequential carry over
// the chunks, then a pass that uses the carries (forward for h; the backward recurrence
//   dh_t = dout_t gelu(y_t) + a_{t+1} dh_{t+1}
// in reverse, re-running the chunk's forward in registers to have h_{t-1}).
#include <math.h>

#include <string.h>

#include <algorithm>

#include "rglru_device.h"
#include "rglru_internal.h"

namespace rglru {
namespace {

constexpr int kBs = 256;    // block size (channels per gate head)
constexpr int kChunk = 64;  // tokens per scan chunk

struct BwdBufs {
    uint16_t *U, *R, *I, *Wt, *dRI, *dRIt, *Ut, *dUg;
    float *aggA, *aggB, *carry, *bP, *bQ, *cin, *duv, *plam, *pba, *pbx, *pconv, *dW, *part;
    size_t part_bytes;
};

size_t r256(size_t n) { return (n + 255) & ~(size_t)255; }

// Carve the workspace (the same order sizes it).
BwdBufs carve(void* ws, int B, int T, int D, int H, size_t* total) {
    const size_t M = (size_t)B * T, MD = M * D, nc = (size_t)B * (T / kChunk) * D;
    char* p = static_cast<char*>(ws);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* q = p ? p + off : nullptr;
        off += r256(bytes);
        return q;
    };
    BwdBufs b;
    b.U = reinterpret_cast<uint16_t*>(take(MD * 2));
    b.R = reinterpret_cast<uint16_t*>(take(MD * 2));
    b.I = reinterpret_cast<uint16_t*>(take(MD * 2));
    b.Wt = reinterpret_cast<uint16_t*>(take((size_t)H * kBs * 2 * kBs * 2));
    b.dRI = reinterpret_cast<uint16_t*>(take(MD * 2 * 2));
    b.dRIt = reinterpret_cast<uint16_t*>(take(MD * 2 * 2));
    b.Ut = reinterpret_cast<uint16_t*>(take(MD * 2));
    b.dUg = reinterpret_cast<uint16_t*>(take(MD * 2));
    b.aggA = reinterpret_cast<float*>(take(nc * 4));
    b.aggB = reinterpret_cast<float*>(take(nc * 4));
    b.carry = reinterpret_cast<float*>(take(nc * 4));
    b.bP = reinterpret_cast<float*>(take(nc * 4));
    b.bQ = reinterpret_cast<float*>(take(nc * 4));
    b.cin = reinterpret_cast<float*>(take(nc * 4));
    b.duv = reinterpret_cast<float*>(take(MD * 4));
    b.plam = reinterpret_cast<float*>(take(nc * 4));
    b.pba = reinterpret_cast<float*>(take(nc * 4));
    b.pbx = reinterpret_cast<float*>(take(nc * 4));
    b.pconv = reinterpret_cast<float*>(take(nc * 5 * 4));
    b.dW = reinterpret_cast<float*>(take((size_t)H * 2 * kBs * kBs * 4));
    b.part_bytes = proj_gemm_part_bytes(2 * kBs, kBs, (int)M);
    b.part = reinterpret_cast<float*>(take(b.part_bytes));
    *total = off;
    return b;
}

__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + expf(-z)); }

__device__ __forceinline__ float gelu_grad(float y) {
    const float k = 0.7978845608028654f;
    const float th = tanhf(k * (y + 0.044715f * y * y * y));
    return 0.5f * (1.0f + th) + 0.5f * y * (1.0f - th * th) * k * (1.0f + 3.0f * 0.044715f * y * y);
}

__device__ __forceinline__ size_t hm(int h, size_t m, int k, size_t M) {
    return ((size_t)h * M + m) * kBs + k;
}

// ---- conv: U (head-major, bf16 as the forward rounds it) -----------------------------------
__global__ void __launch_bounds__(256) bwd_conv_fwd_kernel(BwdArgs a, BwdBufs w) {
    const size_t M = (size_t)a.B * a.T, idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * a.D) return;
    const int d = (int)(idx % a.D);
    const size_t m = idx / a.D;
    const int b = (int)(m / a.T), t = (int)(m % a.T);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* c0 = static_cast<const uint16_t*>(a.conv0);
    const uint16_t* cw = static_cast<const uint16_t*>(a.conv_w);
    float u = a.conv_b ? bf2f(static_cast<const uint16_t*>(a.conv_b)[d]) : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int p = t - 3 + j;
        const float xv = p >= 0 ? bf2f(x[((size_t)b * a.T + p) * a.D + d])
                                : (c0 ? bf2f(c0[((size_t)b * 3 + p + 3) * a.D + d]) : 0.0f);
        u = __builtin_fmaf(bf2f(cw[(size_t)d * 4 + j]), xv, u);
    }
    w.U[hm(d / kBs, m, d % kBs, M)] = f2bf(u);
}

// ---- [W_a^T | W_x^T] per head: Wt[h][k][j'] ------------------------------------------------
__global__ void __launch_bounds__(256) bwd_wtrans_kernel(BwdArgs a, BwdBufs w) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.H * kBs * 2 * kBs) return;
    const int jp = (int)(idx % (2 * kBs)), k = (int)((idx / (2 * kBs)) % kBs);
    const int h = (int)(idx / ((size_t)2 * kBs * kBs));
    const uint16_t* W = static_cast<const uint16_t*>(jp < kBs ? a.wa : a.wx);
    w.Wt[idx] = W[((size_t)h * kBs + (jp % kBs)) * kBs + k];
}

// gate values of one element from the pre-activations
struct Gate {
    float r, i, a, m, lsg;   // lsg = log sigma(Lambda)
};
__device__ __forceinline__ Gate gate_of(float rp, float ip, float lam) {
    Gate g;
    g.r = sigm(rp);
    g.i = sigm(ip);
    g.lsg = -log1pf(expf(-lam));                // log sigma(Lambda)
    const float la = 8.0f * g.r * g.lsg;        // log a
    g.a = expf(la);
    g.m = sqrtf(-expm1f(2.0f * la));            // sqrt(1 - a^2), accurate as a -> 1
    return g;
}

// ---- forward chunk aggregates: (prod a, local h at the chunk end from 0) ------------------
__global__ void __launch_bounds__(256) bwd_scan_agg_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * nch * a.D) return;
    const int d = (int)(idx % a.D), c = (int)((idx / a.D) % nch), b = (int)(idx / ((size_t)nch * a.D));
    const size_t M = (size_t)a.B * a.T;
    const int h = d / kBs, k = d % kBs;
    const float lam = a.lambda[d];
    float A = 1.0f, Bh = 0.0f;
    for (int tt = 0; tt < kChunk; ++tt) {
        const size_t m = (size_t)b * a.T + c * kChunk + tt, e = hm(h, m, k, M);
        const Gate g = gate_of(bf2f(w.R[e]), bf2f(w.I[e]), lam);
        A *= g.a;
        Bh = __builtin_fmaf(g.a, Bh, g.m * g.i * bf2f(w.U[e]));
    }
    w.aggA[idx] = A;
    w.aggB[idx] = Bh;
}

// ---- sequential carries over chunks: h entering each chunk ---------------------------------
__global__ void __launch_bounds__(256) bwd_scan_carry_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * a.D) return;
    const int d = (int)(idx % a.D), b = (int)(idx / a.D);
    float h = a.h0 ? a.h0[idx] : 0.0f;
    for (int c = 0; c < nch; ++c) {
        const size_t e = ((size_t)b * nch + c) * a.D + d;
        w.carry[e] = h;
        h = __builtin_fmaf(w.aggA[e], h, w.aggB[e]);
    }
}

// ---- backward chunk aggregates: c_start = P c_in + Q over the chunk in reverse -------------
// (c_t = a_t dh_t is what token t passes to h_{t-1}; dh_t = dout_t gelu(y_t) + c_{t+1})
__global__ void __launch_bounds__(256) bwd_rscan_agg_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * nch * a.D) return;
    const int d = (int)(idx % a.D), c = (int)((idx / a.D) % nch), b = (int)(idx / ((size_t)nch * a.D));
    const size_t M = (size_t)a.B * a.T;
    const int h = d / kBs, k = d % kBs;
    const float lam = a.lambda[d];
    const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
    const uint16_t* y = static_cast<const uint16_t*>(a.y);
    float P = 1.0f, Q = 0.0f;
    for (int tt = kChunk - 1; tt >= 0; --tt) {
        const size_t m = (size_t)b * a.T + c * kChunk + tt, e = hm(h, m, k, M);
        const Gate g = gate_of(bf2f(w.R[e]), bf2f(w.I[e]), lam);
        const float gt = bf2f(dout[m * a.D + d]) * gelu_precise(bf2f(y[m * a.D + d]));
        Q = g.a * (gt + Q);
        P *= g.a;
    }
    w.bP[idx] = P;
    w.bQ[idx] = Q;
}

__global__ void __launch_bounds__(256) bwd_rscan_carry_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * a.D) return;
    const int d = (int)(idx % a.D), b = (int)(idx / a.D);
    float cc = a.dh_last ? a.dh_last[idx] : 0.0f;
    for (int c = nch - 1; c >= 0; --c) {
        const size_t e = ((size_t)b * nch + c) * a.D + d;
        w.cin[e] = cc;
        cc = __builtin_fmaf(w.bP[e], cc, w.bQ[e]);
    }
    a.dh0[idx] = cc;
}

// ---- per-element gradients of one chunk ----------------------------------------------------
__global__ void __launch_bounds__(256) bwd_grad_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * nch * a.D) return;
    const int d = (int)(idx % a.D), c = (int)((idx / a.D) % nch), b = (int)(idx / ((size_t)nch * a.D));
    const size_t M = (size_t)a.B * a.T;
    const int h = d / kBs, k = d % kBs;
    const float lam = a.lambda[d];
    const float sg = sigm(lam);
    const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
    const uint16_t* y = static_cast<const uint16_t*>(a.y);
    uint16_t* dy = static_cast<uint16_t*>(a.dy);
    const size_t m0 = (size_t)b * a.T + (size_t)c * kChunk;
    // forward within the chunk: h_{t-1} of every token
    float hp[kChunk];
    {
        float hv = w.carry[idx];
#pragma unroll
        for (int tt = 0; tt < kChunk; ++tt) {
            hp[tt] = hv;
            const size_t e = hm(h, m0 + tt, k, M);
            const Gate g = gate_of(bf2f(w.R[e]), bf2f(w.I[e]), lam);
            hv = __builtin_fmaf(g.a, hv, g.m * g.i * bf2f(w.U[e]));
        }
    }
    uint32_t tr[kChunk / 2], ti[kChunk / 2], tu[kChunk / 2];   // transposed rows, bf16 pairs
    float cc = w.cin[idx], slam = 0.0f, sba = 0.0f, sbx = 0.0f;
#pragma unroll
    for (int tt = kChunk - 1; tt >= 0; --tt) {
        const size_t m = m0 + tt, e = hm(h, m, k, M);
        const float u = bf2f(w.U[e]);
        const Gate g = gate_of(bf2f(w.R[e]), bf2f(w.I[e]), lam);
        const float ht = __builtin_fmaf(g.a, hp[tt], g.m * g.i * u);
        const float yv = bf2f(y[m * a.D + d]), dov = bf2f(dout[m * a.D + d]);
        const float dh = __builtin_fmaf(dov, gelu_precise(yv), cc);
        dy[m * a.D + d] = f2bf(dov * ht * gelu_grad(yv));
        w.duv[e] = dh * g.m * g.i;
        const float dm = dh * g.i * u, di = dh * g.m * u;
        const float da = dh * hp[tt] - dm * g.a / g.m;
        slam += da * g.a * 8.0f * g.r * (1.0f - sg);
        const float dr = da * g.a * 8.0f * g.lsg;
        const float dRp = dr * g.r * (1.0f - g.r), dIp = di * g.i * (1.0f - g.i);
        sba += dRp;
        sbx += dIp;
        const uint16_t rb = f2bf(dRp), ib = f2bf(dIp);
        w.dRI[((size_t)h * M + m) * (2 * kBs) + k] = rb;
        w.dRI[((size_t)h * M + m) * (2 * kBs) + kBs + k] = ib;
        const uint32_t ub = w.U[e];
        if (tt & 1) {
            tr[tt / 2] = (uint32_t)rb << 16;
            ti[tt / 2] = (uint32_t)ib << 16;
            tu[tt / 2] = ub << 16;
        } else {
            tr[tt / 2] |= rb;
            ti[tt / 2] |= ib;
            tu[tt / 2] |= ub;
        }
        cc = dh * g.a;
    }
    // token-contiguous rows for the weight-gradient GEMM: 128 bytes per lane and array
    uint4* dr_t = reinterpret_cast<uint4*>(w.dRIt + ((size_t)h * 2 * kBs + k) * M + m0);
    uint4* di_t = reinterpret_cast<uint4*>(w.dRIt + ((size_t)h * 2 * kBs + kBs + k) * M + m0);
    uint4* u_t = reinterpret_cast<uint4*>(w.Ut + ((size_t)h * kBs + k) * M + m0);
#pragma unroll
    for (int q = 0; q < kChunk / 8; ++q) {
        dr_t[q] = make_uint4(tr[4 * q], tr[4 * q + 1], tr[4 * q + 2], tr[4 * q + 3]);
        di_t[q] = make_uint4(ti[4 * q], ti[4 * q + 1], ti[4 * q + 2], ti[4 * q + 3]);
        u_t[q] = make_uint4(tu[4 * q], tu[4 * q + 1], tu[4 * q + 2], tu[4 * q + 3]);
    }
    w.plam[idx] = slam;
    w.pba[idx] = sba;
    w.pbx[idx] = sbx;
}

// ---- conv backward: dx, the conv0 window, per-chunk partial sums of the conv weights -------
__global__ void __launch_bounds__(256) bwd_conv_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * nch * a.D) return;
    const int d = (int)(idx % a.D), c = (int)((idx / a.D) % nch), b = (int)(idx / ((size_t)nch * a.D));
    const size_t M = (size_t)a.B * a.T;
    const int h = d / kBs, k = d % kBs;
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* c0 = static_cast<const uint16_t*>(a.conv0);
    const uint16_t* cw = static_cast<const uint16_t*>(a.conv_w);
    uint16_t* dx = static_cast<uint16_t*>(a.dx);
    float wj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wj[j] = bf2f(cw[(size_t)d * 4 + j]);
    auto dU = [&](int t) -> float {   // total gradient of u at token t of sequence b (0 past T)
        if (t >= a.T) return 0.0f;
        const size_t e = hm(h, (size_t)b * a.T + t, k, M);
        return w.duv[e] + bf2f(w.dUg[e]);
    };
    auto xt = [&](int p) -> float {   // x~ at position p (negative: the conv0 window)
        if (p >= 0) return bf2f(x[((size_t)b * a.T + p) * a.D + d]);
        return c0 ? bf2f(c0[((size_t)b * 3 + p + 3) * a.D + d]) : 0.0f;
    };
    const int t0 = c * kChunk;
    float g0 = dU(t0), g1 = dU(t0 + 1), g2 = dU(t0 + 2);
    float sw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sb = 0.0f;
    for (int tt = 0; tt < kChunk; ++tt) {
        const int t = t0 + tt;
        const float g3 = dU(t + 3);
        // u_t takes x~_{t-3+j} with tap j, so x_t feeds u_{t+3-j} through tap j
        dx[((size_t)b * a.T + t) * a.D + d] =
            f2bf(wj[3] * g0 + wj[2] * g1 + wj[1] * g2 + wj[0] * g3);
        sb += g0;
#pragma unroll
        for (int j = 0; j < 4; ++j) sw[j] = __builtin_fmaf(g0, xt(t - 3 + j), sw[j]);
        g0 = g1;
        g1 = g2;
        g2 = g3;
    }
    float* pc = w.pconv + idx * 5;
    pc[0] = sw[0]; pc[1] = sw[1]; pc[2] = sw[2]; pc[3] = sw[3]; pc[4] = sb;
    if (c == 0) {
        // window slot s (position s - 3) feeds u_t through tap j = s - t for t = 0 .. s
        for (int s = 0; s < 3; ++s) {
            float v = 0.0f;
            for (int t = 0; t <= s && t < a.T; ++t) v = __builtin_fmaf(wj[s - t], dU(t), v);
            a.dconv0[((size_t)b * 3 + s) * a.D + d] = v;
        }
    }
}

// ---- fixed-order sums of the partials; dW from the GEMM's fp32 output ----------------------
__global__ void __launch_bounds__(256) bwd_reduce_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t nw = (size_t)a.H * kBs * kBs;
    if (idx < nw) {   // [H][2 bs][bs] -> dwa, dwx
        const size_t h = idx / ((size_t)kBs * kBs), r = idx % ((size_t)kBs * kBs);
        a.dwa[idx] = w.dW[h * 2 * kBs * kBs + r];
        a.dwx[idx] = w.dW[h * 2 * kBs * kBs + (size_t)kBs * kBs + r];
    }
    if (idx >= (size_t)a.D) return;
    const int d = (int)idx;
    float sl = 0.0f, sa = 0.0f, sx = 0.0f, sw[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int b = 0; b < a.B; ++b)
        for (int c = 0; c < nch; ++c) {
            const size_t e = ((size_t)b * nch + c) * a.D + d;
            sl += w.plam[e];
            sa += w.pba[e];
            sx += w.pbx[e];
#pragma unroll
            for (int j = 0; j < 5; ++j) sw[j] += w.pconv[e * 5 + j];
        }
    a.dlambda[d] = sl;
    a.dba[d] = sa;
    a.dbx[d] = sx;
#pragma unroll
    for (int j = 0; j < 4; ++j) a.dconv_w[(size_t)d * 4 + j] = sw[j];
    a.dconv_b[d] = sw[4];
}

unsigned blocks_for(size_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

size_t backward_workspace_bytes(int B, int T, int D, int H) {
    size_t total = 0;
    carve(nullptr, B, T, D, H, &total);
    return total;
}

hipError_t launch_prefill_backward(const BwdArgs& a, hipStream_t s) {
    size_t total = 0;
    const BwdBufs w = carve(a.ws, a.B, a.T, a.D, a.H, &total);
    const size_t M = (size_t)a.B * a.T, nch = a.T / kChunk;
    const size_t nlane = (size_t)a.B * nch * a.D;
    hipError_t e;
#define RG_LAUNCH(kern, n)                                                              \
    hipLaunchKernelGGL(kern, dim3(blocks_for(n)), dim3(256), 0, s, a, w);               \
    if ((e = hipGetLastError()) != hipSuccess) return e;
    RG_LAUNCH(bwd_conv_fwd_kernel, M * a.D);
    RG_LAUNCH(bwd_wtrans_kernel, (size_t)a.H * kBs * 2 * kBs);
    for (int h = 0; h < a.H; ++h) {   // gate pre-activations
        ProjGemmArgs g;
        memset(&g, 0, sizeof g);
        g.A = w.U + (size_t)h * M * kBs;
        g.W[0] = static_cast<const uint16_t*>(a.wa) + (size_t)h * kBs * kBs;
        g.W[1] = static_cast<const uint16_t*>(a.wx) + (size_t)h * kBs * kBs;
        g.b[0] = a.ba ? static_cast<const uint16_t*>(a.ba) + (size_t)h * kBs : nullptr;
        g.b[1] = a.bx ? static_cast<const uint16_t*>(a.bx) + (size_t)h * kBs : nullptr;
        g.C[0] = w.R + (size_t)h * M * kBs;
        g.C[1] = w.I + (size_t)h * M * kBs;
        g.Nw[0] = kBs; g.Nw[1] = kBs; g.nseg = 2; g.M = (int)M; g.K = kBs;
        if ((e = launch_proj_gemm(g, s)) != hipSuccess) return e;
    }
    RG_LAUNCH(bwd_scan_agg_kernel, nlane);
    RG_LAUNCH(bwd_scan_carry_kernel, (size_t)a.B * a.D);
    RG_LAUNCH(bwd_rscan_agg_kernel, nlane);
    RG_LAUNCH(bwd_rscan_carry_kernel, (size_t)a.B * a.D);
    RG_LAUNCH(bwd_grad_kernel, nlane);
    for (int h = 0; h < a.H; ++h) {   // gradient of u through the gates
        ProjGemmArgs g;
        memset(&g, 0, sizeof g);
        g.A = w.dRI + (size_t)h * M * 2 * kBs;
        g.W[0] = w.Wt + (size_t)h * kBs * 2 * kBs;
        g.C[0] = w.dUg + (size_t)h * M * kBs;
        g.Nw[0] = kBs; g.nseg = 1; g.M = (int)M; g.K = 2 * kBs;
        if ((e = launch_proj_gemm(g, s)) != hipSuccess) return e;
    }
    for (int h = 0; h < a.H; ++h) {   // gate weight gradients (K = B * T, fp32)
        ProjGemmArgs g;
        memset(&g, 0, sizeof g);
        g.A = w.dRIt + (size_t)h * 2 * kBs * M;
        g.W[0] = w.Ut + (size_t)h * kBs * M;
        g.C[0] = w.dW + (size_t)h * 2 * kBs * kBs;
        g.Nw[0] = kBs; g.nseg = 1; g.M = 2 * kBs; g.K = (int)M;
        g.part = w.part; g.part_bytes = w.part_bytes; g.c_f32 = 1;
        if ((e = launch_proj_gemm(g, s)) != hipSuccess) return e;
    }
    RG_LAUNCH(bwd_conv_kernel, nlane);
    RG_LAUNCH(bwd_reduce_kernel, std::max((size_t)a.D, (size_t)a.H * kBs * kBs));
#undef RG_LAUNCH
    return hipSuccess;
}

}  // namespace rglru
