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
// The scans run per channel over chunks of 32 tokens: local aggregates of both directions in one
// pass, sequential carries over the chunks, then a pass that uses the carries (forward for h; the backward recurrence
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
constexpr int kChunk = 32;  // tokens per scan chunk (32: the gradient pass keeps a chunk in registers)

struct BwdBufs {
    uint16_t *U, *R, *I, *Wt, *dRI, *dRIt, *Ut, *dUg;
    float *aggA, *aggB, *carry, *bQ, *cin, *duv, *plam, *pba, *pbx, *pconv, *dW, *part;
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

// sigmoid with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float sigm(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// gelu_tanh(y) and its derivative from one tanh
__device__ __forceinline__ float2 gelu_and_grad(float y) {
    const float k = 0.7978845608028654f;
    const float th = tanhf(k * (y + 0.044715f * y * y * y));
    return make_float2(0.5f * y * (1.0f + th),
                       0.5f * (1.0f + th) +
                           0.5f * y * (1.0f - th * th) * k * (1.0f + 3.0f * 0.044715f * y * y));
}

__device__ __forceinline__ size_t hm(int h, size_t m, int k, size_t M) {
    return ((size_t)h * M + m) * kBs + k;
}

// ---- conv: U (head-major, bf16 as the forward rounds it); eight channels per thread --------
__device__ __forceinline__ void unpack8(uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = bf_lo(w[q]);
        f[2 * q + 1] = bf_hi(w[q]);
    }
}

__global__ void __launch_bounds__(256) bwd_conv_fwd_kernel(BwdArgs a, BwdBufs w) {
    // grid: (B * T token rows, D / 2048 channel blocks); thread: channels d .. d + 7
    const size_t M = (size_t)a.B * a.T;
    const int d = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (d >= a.D) return;
    const size_t m = blockIdx.x;
    const int b = (int)(m / a.T), t = (int)(m % a.T);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* c0 = static_cast<const uint16_t*>(a.conv0);
    const uint4* cw = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.conv_w) + (size_t)d * 4);
    float u[8], wt[32];
    if (a.conv_b) unpack8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.conv_b) + d), u);
    else
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack8(cw[q], wt + 8 * q);   // wt[4 c + j]: channel d + c, tap j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int p = t - 3 + j;
        float xv[8];
        if (p >= 0) unpack8(*reinterpret_cast<const uint4*>(x + ((size_t)b * a.T + p) * a.D + d), xv);
        else if (c0) unpack8(*reinterpret_cast<const uint4*>(c0 + ((size_t)b * 3 + p + 3) * a.D + d), xv);
        else
#pragma unroll
            for (int q = 0; q < 8; ++q) xv[q] = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = __builtin_fmaf(wt[4 * q + j], xv[q], u[q]);
    }
    *reinterpret_cast<uint4*>(w.U + hm(d / kBs, m, d % kBs, M)) =
        make_uint4(pack2bf(u[0], u[1]), pack2bf(u[2], u[3]), pack2bf(u[4], u[5]), pack2bf(u[6], u[7]));
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

// gate values of one element from the pre-activations; lsg = log sigma(Lambda) of the channel
struct Gate {
    float r, i, a, m;
};
__device__ __forceinline__ Gate gate_of(float rp, float ip, float lsg) {
    Gate g;
    g.r = sigm(rp);
    g.i = sigm(ip);
    const float la = 8.0f * g.r * lsg;          // log a
    g.a = __builtin_amdgcn_exp2f(la * kLog2e);
    g.m = sqrtf(-expm1f(2.0f * la));            // sqrt(1 - a^2), accurate as a -> 1
    return g;
}
__device__ __forceinline__ float log_sigmoid(float lam) { return -log1pf(expf(-lam)); }

// ---- chunk aggregates, both directions in one forward pass over the chunk -----------------
// forward: h_end = A h_start + Bh with A = prod a, Bh the local state from 0;
// reverse: c_start = A c_in + Q with c_t = a_t dh_t, dh_t = dout_t gelu(y_t) + c_{t+1}, i.e.
// Q = sum_t (a_start ... a_t) dout_t gelu(y_t).
__global__ void __launch_bounds__(256) bwd_chunk_agg_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * nch * a.D) return;
    const int d = (int)(idx % a.D), c = (int)((idx / a.D) % nch), b = (int)(idx / ((size_t)nch * a.D));
    const size_t M = (size_t)a.B * a.T;
    const int h = d / kBs, k = d % kBs;
    const float lsg = log_sigmoid(a.lambda[d]);
    const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
    const uint16_t* y = static_cast<const uint16_t*>(a.y);
    float A = 1.0f, Bh = 0.0f, Q = 0.0f;
    for (int tt = 0; tt < kChunk; ++tt) {
        const size_t m = (size_t)b * a.T + c * kChunk + tt, e = hm(h, m, k, M);
        const Gate g = gate_of(bf2f(w.R[e]), bf2f(w.I[e]), lsg);
        A *= g.a;
        Bh = __builtin_fmaf(g.a, Bh, g.m * g.i * bf2f(w.U[e]));
        Q = __builtin_fmaf(A, bf2f(dout[m * a.D + d]) * gelu_and_grad(bf2f(y[m * a.D + d])).x, Q);
    }
    w.aggA[idx] = A;
    w.aggB[idx] = Bh;
    w.bQ[idx] = Q;
}

// ---- sequential carries over the chunks: h entering each chunk (forward) and c entering it
// from the right (reverse); the reverse carry past the first chunk is dh0 ----------------------
__global__ void __launch_bounds__(256) bwd_carry_kernel(BwdArgs a, BwdBufs w) {
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
    float cc = a.dh_last ? a.dh_last[idx] : 0.0f;
    for (int c = nch - 1; c >= 0; --c) {
        const size_t e = ((size_t)b * nch + c) * a.D + d;
        w.cin[e] = cc;
        cc = __builtin_fmaf(w.aggA[e], cc, w.bQ[e]);
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
    const float lsg = log_sigmoid(a.lambda[d]);
    const float sg = expf(lsg);
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
            const Gate g = gate_of(bf2f(w.R[e]), bf2f(w.I[e]), lsg);
            hv = __builtin_fmaf(g.a, hv, g.m * g.i * bf2f(w.U[e]));
        }
    }
    uint32_t tr[kChunk / 2], ti[kChunk / 2], tu[kChunk / 2];   // transposed rows, bf16 pairs
    float cc = w.cin[idx], slam = 0.0f, sba = 0.0f, sbx = 0.0f;
#pragma unroll
    for (int tt = kChunk - 1; tt >= 0; --tt) {
        const size_t m = m0 + tt, e = hm(h, m, k, M);
        const float u = bf2f(w.U[e]);
        const Gate g = gate_of(bf2f(w.R[e]), bf2f(w.I[e]), lsg);
        const float ht = __builtin_fmaf(g.a, hp[tt], g.m * g.i * u);
        const float yv = bf2f(y[m * a.D + d]), dov = bf2f(dout[m * a.D + d]);
        const float2 gg = gelu_and_grad(yv);
        const float dh = __builtin_fmaf(dov, gg.x, cc);
        dy[m * a.D + d] = f2bf(dov * ht * gg.y);
        w.duv[e] = dh * g.m * g.i;
        const float dm = dh * g.i * u, di = dh * g.m * u;
        const float da = dh * hp[tt] - dm * g.a / g.m;
        slam += da * g.a * 8.0f * g.r * (1.0f - sg);
        const float dr = da * g.a * 8.0f * lsg;
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
    // token-contiguous rows for the weight-gradient GEMM: 64 bytes per lane and array
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
// One thread per (sequence, chunk, eight channels), the chunk's tokens in order.
__global__ void __launch_bounds__(256) bwd_conv_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk, D8 = a.D / 8;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * nch * D8) return;
    const int d = (int)(idx % D8) * 8, c = (int)((idx / D8) % nch), b = (int)(idx / ((size_t)nch * D8));
    const size_t M = (size_t)a.B * a.T;
    const int h = d / kBs, k = d % kBs;
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* c0 = static_cast<const uint16_t*>(a.conv0);
    uint16_t* dx = static_cast<uint16_t*>(a.dx);
    float wt[32];   // wt[4 q + j]: channel d + q, tap j
    {
        const uint4* cw = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.conv_w) + (size_t)d * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) unpack8(cw[q], wt + 8 * q);
    }
    auto dU = [&](int t, float* g) {   // total gradient of u at token t (zero past T)
        if (t >= a.T) {
#pragma unroll
            for (int q = 0; q < 8; ++q) g[q] = 0.0f;
            return;
        }
        const size_t e = hm(h, (size_t)b * a.T + t, k, M);
        const float4 v0 = *reinterpret_cast<const float4*>(w.duv + e);
        const float4 v1 = *reinterpret_cast<const float4*>(w.duv + e + 4);
        float ug[8];
        unpack8(*reinterpret_cast<const uint4*>(w.dUg + e), ug);
        g[0] = v0.x + ug[0]; g[1] = v0.y + ug[1]; g[2] = v0.z + ug[2]; g[3] = v0.w + ug[3];
        g[4] = v1.x + ug[4]; g[5] = v1.y + ug[5]; g[6] = v1.z + ug[6]; g[7] = v1.w + ug[7];
    };
    auto xt = [&](int p, float* f) {   // x~ at position p (negative: the conv0 window)
        if (p >= 0) unpack8(*reinterpret_cast<const uint4*>(x + ((size_t)b * a.T + p) * a.D + d), f);
        else if (c0) unpack8(*reinterpret_cast<const uint4*>(c0 + ((size_t)b * 3 + p + 3) * a.D + d), f);
        else
#pragma unroll
            for (int q = 0; q < 8; ++q) f[q] = 0.0f;
    };
    const int t0 = c * kChunk;
    float g[4][8];   // dU at t, t + 1, t + 2, t + 3 (rotating)
    dU(t0, g[0]);
    dU(t0 + 1, g[1]);
    dU(t0 + 2, g[2]);
    float sw[8][4] = {}, sb[8] = {};
    float xw[4][8];  // x~ at t - 3 .. t
    xt(t0 - 3, xw[0]);
    xt(t0 - 2, xw[1]);
    xt(t0 - 1, xw[2]);
#pragma unroll 4
    for (int tt = 0; tt < kChunk; ++tt) {   // by 4: the ring slots become compile-time indices
        const int t = t0 + tt, r = tt & 3;
        // slots: g[(r + i) & 3] holds dU(t + i); xw[(r + j) & 3] holds x~(t - 3 + j)
        dU(t + 3, g[(r + 3) & 3]);
        xt(t, xw[(r + 3) & 3]);
        float o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            // u_t takes x~_{t-3+j} with tap j, so x_t feeds u_{t+3-j} through tap j
            o[q] = wt[4 * q + 3] * g[r][q] + wt[4 * q + 2] * g[(r + 1) & 3][q] +
                   wt[4 * q + 1] * g[(r + 2) & 3][q] + wt[4 * q] * g[(r + 3) & 3][q];
            sb[q] += g[r][q];
#pragma unroll
            for (int j = 0; j < 4; ++j) sw[q][j] = __builtin_fmaf(g[r][q], xw[(r + j) & 3][q], sw[q][j]);
        }
        *reinterpret_cast<uint4*>(dx + ((size_t)b * a.T + t) * a.D + d) =
            make_uint4(pack2bf(o[0], o[1]), pack2bf(o[2], o[3]), pack2bf(o[4], o[5]), pack2bf(o[6], o[7]));
    }
    const size_t pe = ((size_t)b * nch + c) * a.D + d;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        float* pc = w.pconv + (pe + q) * 5;
        pc[0] = sw[q][0]; pc[1] = sw[q][1]; pc[2] = sw[q][2]; pc[3] = sw[q][3]; pc[4] = sb[q];
    }
    if (c == 0) {
        // window slot s (position s - 3) feeds u_t through tap j = s - t for t = 0 .. s
        float gg[3][8];
        dU(0, gg[0]);
        dU(1, gg[1]);
        dU(2, gg[2]);
        for (int s2 = 0; s2 < 3; ++s2)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float v = 0.0f;
                for (int t = 0; t <= s2 && t < a.T; ++t) v = __builtin_fmaf(wt[4 * q + s2 - t], gg[t][q], v);
                a.dconv0[((size_t)b * 3 + s2) * a.D + d + q] = v;
            }
    }
}

// ---- fixed-order sums of the partials; dW from the GEMM's fp32 output ----------------------
__global__ void __launch_bounds__(256) bwd_wcopy_kernel(BwdArgs a, BwdBufs w) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.H * kBs * kBs) return;   // [H][2 bs][bs] -> dwa, dwx
    const size_t h = idx / ((size_t)kBs * kBs), r = idx % ((size_t)kBs * kBs);
    a.dwa[idx] = w.dW[h * 2 * kBs * kBs + r];
    a.dwx[idx] = w.dW[h * 2 * kBs * kBs + (size_t)kBs * kBs + r];
}

// One wave per channel: lane l sums partials l, l + 64, ... in order, then a fixed butterfly.
__global__ void __launch_bounds__(256) bwd_reduce_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk, np = a.B * nch;
    const int d = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (d >= a.D) return;
    float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int q = lane; q < np; q += 64) {
        const size_t e = (size_t)q * a.D + d;
        v[0] += w.plam[e];
        v[1] += w.pba[e];
        v[2] += w.pbx[e];
#pragma unroll
        for (int j = 0; j < 5; ++j) v[3 + j] += w.pconv[e * 5 + j];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] += __shfl_xor(v[j], o);
    if (lane != 0) return;
    a.dlambda[d] = v[0];
    a.dba[d] = v[1];
    a.dbx[d] = v[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) a.dconv_w[(size_t)d * 4 + j] = v[3 + j];
    a.dconv_b[d] = v[7];
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
    hipLaunchKernelGGL(bwd_conv_fwd_kernel, dim3((unsigned)M, (unsigned)((a.D / 8 + 255) / 256)),
                       dim3(256), 0, s, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
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
    RG_LAUNCH(bwd_chunk_agg_kernel, nlane);
    RG_LAUNCH(bwd_carry_kernel, (size_t)a.B * a.D);
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
    RG_LAUNCH(bwd_conv_kernel, nlane / 8);
    RG_LAUNCH(bwd_wcopy_kernel, (size_t)a.H * kBs * kBs);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((a.D + 3) / 4)), dim3(256), 0, s, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
#undef RG_LAUNCH
    return hipSuccess;
}

}  // namespace rglru
