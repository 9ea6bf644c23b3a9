// Backward pass of the recurrent block's temporal-mixing path, for gfx950 (CDNA4).  The pages
// give no training detail; these are the chain-rule gradients of the forward definition
// (conv k=4 -> block-diagonal gates -> RG-LRU -> times GELU-tanh of y) for
//   L = sum_t dout_t . out_t + dh_last . h_{T-1}.
//
// Intermediates are head-major, [H][B*T][256] (channel k of head h of token m at
// (h * M + m) * 256 + k).  The three block-diagonal products:
//   gates:      [Rpre | Ipre]_h = U_h [W_a[h]; W_x[h]]^T + b           (K = 256)
//   input grad: dU_h = [dRpre | dIpre]_h [W_a[h]^T | W_x[h]^T]^T       (K = 512)
//   weights:    [dW_a; dW_x]_h = [dRpre | dIpre]_h^T U_h                (K = B*T, split K, fp32)
// The first runs inside the front pass (conv, gates on MFMA with the weights held in registers,
// chunk aggregates); the input gradient is a persistent kernel of the same kind (the transposed
// weights held in registers); the weight gradients have a kernel of their own that reads dRI and
// U in their head-major layout (K runs over tokens).  The scans run per channel over chunks of 32 tokens: local
// aggregates of both directions (front pass), sequential carries over the chunks, then a pass
// that uses the carries (forward for h; the backward recurrence
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
    uint16_t *U, *R, *I, *Wt, *dRI, *dUg;
    float *aggA, *aggB, *carry, *bQ, *cin, *duv, *plam, *pba, *pbx, *pconv, *wpart;
    float *sA, *sB, *sQ, *sh, *sc;   // chunk-group aggregates and carries (two-level carry scan)
    float* red;                       // reduction parts [kRedParts][8][D]
    int wsplits;                      // token splits of the weight-gradient product
};

size_t r256(size_t n) { return (n + 255) & ~(size_t)255; }

// the carry scan over a sequence's nch chunks runs in groups of kGroupChunks consecutive chunks
constexpr int kGroupChunks = 16;
__host__ __device__ inline int groups_of(int nch) { return (nch + kGroupChunks - 1) / kGroupChunks; }
// the fixed-order sums of the per-chunk partials run in kRedParts consecutive ranges
constexpr int kRedParts = 32;

// The weight-gradient product splits the B*T tokens into this many ranges (about one
// workgroup per CU over the 2 H output tiles; each range one 32-token step at least); its
// fp32 partials are summed in range order.
constexpr int kWgSplitMax = 16;
inline int wgrad_splits(int B, int T, int H) {
    const int ksteps = (int)((long long)B * T / 32);
    return std::max(1, std::min(std::min(ksteps, kWgSplitMax), 256 / (2 * H)));
}

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
    b.pconv = reinterpret_cast<float*>(take(nc * 5 * 4));   // [5][B * nch * D]
    const size_t ng = (size_t)B * groups_of(T / kChunk) * D;
    b.sA = reinterpret_cast<float*>(take(ng * 4));
    b.sB = reinterpret_cast<float*>(take(ng * 4));
    b.sQ = reinterpret_cast<float*>(take(ng * 4));
    b.sh = reinterpret_cast<float*>(take(ng * 4));
    b.sc = reinterpret_cast<float*>(take(ng * 4));
    b.red = reinterpret_cast<float*>(take((size_t)kRedParts * 8 * D * 4));
    b.wsplits = wgrad_splits(B, T, H);
    b.wpart = reinterpret_cast<float*>(take((size_t)b.wsplits * H * 2 * kBs * kBs * 4));
    *total = off;
    return b;
}

// sigmoid with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float sigm(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// gelu_tanh(y) and its derivative from one exponential: with z = k (y + c y^3),
// 0.5 (1 + tanh z) = s = 1 / (1 + e^(-2z)), so gelu = y s and
// gelu' = s + y s (1 - s) 2k (1 + 3c y^2); hardware exp2 and reciprocal (about 1 ulp each;
// s saturates to 0 or 1 for large |z|)
__device__ __forceinline__ float2 gelu_and_grad(float y) {
    constexpr float k = 0.7978845608028654f, c = 0.044715f;
    const float y2 = y * y;
    const float e = __builtin_amdgcn_exp2f(y * __builtin_fmaf(y2, -2.0f * k * c * kLog2e, -2.0f * k * kLog2e));
    const float sv = __builtin_amdgcn_rcpf(1.0f + e);
    const float gx = y * sv;
    return make_float2(gx, __builtin_fmaf(gx * (1.0f - sv), __builtin_fmaf(y2, 6.0f * k * c, 2.0f * k), sv));
}

// sqrt(1 - a^2) from x = 2 log a <= 0 and a = e^(x/2): 1 - e^x by its degree-7 Taylor
// polynomial above x = -0.5 (full relative accuracy as a -> 1; truncation below 1e-7
// relative), 1 - a a below it (no cancellation there)
__device__ __forceinline__ float sqrt_one_minus_a2(float x, float av) {
    float p = __builtin_fmaf(x, 1.0f / 5040.0f, 1.0f / 720.0f);
    p = __builtin_fmaf(x, p, 1.0f / 120.0f);
    p = __builtin_fmaf(x, p, 1.0f / 24.0f);
    p = __builtin_fmaf(x, p, 1.0f / 6.0f);
    p = __builtin_fmaf(x, p, 0.5f);
    p = __builtin_fmaf(x, p, 1.0f);
    return __builtin_amdgcn_sqrtf(x > -0.5f ? -x * p : __builtin_fmaf(-av, av, 1.0f));
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


// ---- [W_a^T | W_x^T] per head: Wt[h][k][j'] ------------------------------------------------
__global__ void __launch_bounds__(256) bwd_wtrans_kernel(BwdArgs a, BwdBufs w) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.H * kBs * 2 * kBs) return;
    const int jp = (int)(idx % (2 * kBs)), k = (int)((idx / (2 * kBs)) % kBs);
    const int h = (int)(idx / ((size_t)2 * kBs * kBs));
    const uint16_t* W = static_cast<const uint16_t*>(jp < kBs ? a.wa : a.wx);
    w.Wt[idx] = W[((size_t)h * kBs + (jp % kBs)) * kBs + k];
}

// gate values of one element from the pre-activations; lsg = log sigma(Lambda) of the channel.
// (The front pass's form: sqrt(1 - a^2) as sqrt(1 - e^(2 log a)) throughout, its large-x side
// with a second exponential; 1 - a a there, as in the gradient pass, costs the front pass
// register spills.)
struct Gate {
    float r, i, a, m;
};
__device__ __forceinline__ Gate gate_of(float rp, float ip, float lsg) {
    Gate g;
    g.r = sigm(rp);
    g.i = sigm(ip);
    const float la = 8.0f * g.r * lsg;          // log a
    g.a = __builtin_amdgcn_exp2f(la * kLog2e);
    const float x = 2.0f * la;
    float p = __builtin_fmaf(x, 1.0f / 5040.0f, 1.0f / 720.0f);
    p = __builtin_fmaf(x, p, 1.0f / 120.0f);
    p = __builtin_fmaf(x, p, 1.0f / 24.0f);
    p = __builtin_fmaf(x, p, 1.0f / 6.0f);
    p = __builtin_fmaf(x, p, 0.5f);
    p = __builtin_fmaf(x, p, 1.0f);
    const float small = -x * p;
    const float large = 1.0f - __builtin_amdgcn_exp2f(x * kLog2e);
    g.m = __builtin_amdgcn_sqrtf(x > -0.5f ? small : large);
    return g;
}
__device__ __forceinline__ float log_sigmoid(float lam) { return -log1pf(expf(-lam)); }

// Per-token accesses of the scan kernels go through buffer resources based at the block's first
// token (the block's sequence, chunk and head are uniform): a lane's channel is its 32-bit
// offset and a token's stride a scalar offset, so no 64-bit address is formed per access.
// The gradient pass also copies whole tiles into LDS through them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffffu, 0x00020000);
}
__device__ __forceinline__ float ld_bf(__amdgpu_buffer_rsrc_t r, int vo, int so) {
    return bf2f((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0));
}
__device__ __forceinline__ void st_f32(__amdgpu_buffer_rsrc_t r, int vo, int so, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, vo, so, 0);
}

// Block decomposition of the scan kernels: one block of kBs lanes per (sequence, chunk, head),
// lane = channel of the head; blockIdx = (b * nch + c) * H + h.
struct ScanBlock {
    int b, c, h;
    size_t m0;   // first token of the chunk
};
__device__ __forceinline__ ScanBlock scan_block(const BwdArgs& a) {
    const int nch = a.T / kChunk;
    ScanBlock s;
    s.h = (int)(blockIdx.x % (unsigned)a.H);
    const unsigned bc = blockIdx.x / (unsigned)a.H;
    s.c = (int)(bc % (unsigned)nch);
    s.b = (int)(bc / (unsigned)nch);
    s.m0 = (size_t)s.b * a.T + (size_t)s.c * kChunk;
    return s;
}


// ---- front pass: conv, gate pre-activations and chunk aggregates in one persistent kernel ----
// One workgroup of eight waves per CU, pinned to a gate head: wave w keeps the MFMA B fragments
// of output channels [32w, 32w + 32) of both gate blocks in VGPRs for the kernel's lifetime, so
// the head's 256 KB of gate weights are read once per workgroup instead of once per output
// tile.  The workgroup walks units of 64 tokens of one sequence (two scan chunks):
//   1. global -> LDS copies of the unit's x rows (with the 3-token halo from the previous tokens,
//      the conv0 window or zeros), and of y and dout rows of each wave's 32 channels;
//   2. conv (fp32, taps in order from the bias, as the per-token definition adds them), u rounded
//      to bf16 into an LDS tile and out to U;
//   3. both gates' pre-activations on MFMA (v_mfma_f32_32x32x16_bf16, K in natural order), tile
//      rows permuted so that each lane holds 32 consecutive tokens of one channel: the low
//      half-wave chunk 0 of the unit, the high half-wave chunk 1;
//   4. per lane: R and I = bias + product rounded to bf16 (as stored), then the chunk's forward
//      aggregate (prod a, local state from 0) and reverse aggregate Q from the rounded values,
//      in token order.
// Outputs: U, R, I head-major and the aggregates, exactly as the separate conv, GEMM and
// aggregate passes would produce them.
constexpr int kFSeg = 64;                  // tokens per unit
constexpr int kFWaves = 8;
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFRow = kBs + 8;             // u row stride (elements)
constexpr int kFXRows = 20;                // x rows of a wave: tokens 16 tg - 3 .. 16 tg + 16
constexpr int kFXElems = kFXRows * 128;
constexpr int kFYElems = kFSeg * 32 + 32;  // y (or dout) rows of a wave's 32 channels

// u row of token t (0..63): tokens 32..63 have row bits 2..3 flipped, so the A-fragment reads of
// tokens t and t + 32 in one pass fall in different bank groups
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int f_urow(int t) { return t ^ (((t >> 5) & 1) * 12); }
// y / dout row r of a wave's region: rows 32..63 start 64 bytes later (the two half-waves'
// 2-byte reads of rows r and r + 32 then fall in different banks)
__device__ __forceinline__ int f_yrow(int r) { return r * 32 + ((r >> 5) << 5); }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_len(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// A copy the compiler cannot see through: addresses derived from it inside the unit loop are
// formed there (one base plus constant offsets) instead of being hoisted out of the loop for
// every token, which would not fit beside the gate weights held in registers.
__device__ __forceinline__ int f_opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ void f_wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
__device__ __forceinline__ void f_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ void __launch_bounds__(kFThreads) bwd_front_kernel(BwdArgs a, BwdBufs w, int wph) {
    __shared__ __attribute__((aligned(16))) uint16_t u_lds[kFSeg * kFRow];
    __shared__ __attribute__((aligned(16))) uint16_t x_lds[kFWaves * kFXElems];
    __shared__ __attribute__((aligned(16))) uint16_t y_lds[kFWaves * kFYElems];
    __shared__ __attribute__((aligned(16))) uint16_t d_lds[kFWaves * kFYElems];
    __shared__ __attribute__((aligned(16))) float4 ctap[kBs];   // conv taps of a channel, fp32
    __shared__ float cbias[kBs], gba[kBs], gbx[kBs], glsg[kBs];
    const uint32_t* const x_lds32 = reinterpret_cast<const uint32_t*>(x_lds);
    uint32_t* const u_lds32 = reinterpret_cast<uint32_t*>(u_lds);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // placement: workgroups are dealt to the 8 XCDs round-robin; consecutive slots of one XCD
    // serve one head, so each XCD's L2 holds few heads' inputs
    const unsigned G = gridDim.x, bid = blockIdx.x;
    const unsigned xcd = bid & 7u, jx = bid >> 3, per = G >> 3, rem = G & 7u;
    const unsigned slot = xcd * per + min(xcd, rem) + jx;
    const int head = (int)(slot / (unsigned)wph), jw = (int)(slot % (unsigned)wph);
    if (head >= a.H) return;
    const int B = a.B, T = a.T, D = a.D;
    const size_t M = (size_t)B * T;
    const int nseg = (T + kFSeg - 1) / kFSeg, nch = T / kChunk;
    const int units = B * nseg;

    for (int i = tid; i < kBs; i += kFThreads) {
        const int d = head * kBs + i;
        float t4[4];
        const uint16_t* cw = static_cast<const uint16_t*>(a.conv_w) + (size_t)d * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) t4[j] = bf2f(cw[j]);
        ctap[i] = make_float4(t4[0], t4[1], t4[2], t4[3]);
        cbias[i] = a.conv_b ? bf2f(static_cast<const uint16_t*>(a.conv_b)[d]) : 0.0f;
        gba[i] = a.ba ? bf2f(static_cast<const uint16_t*>(a.ba)[d]) : 0.0f;
        gbx[i] = a.bx ? bf2f(static_cast<const uint16_t*>(a.bx)[d]) : 0.0f;
        glsg[i] = log_sigmoid(a.lambda[d]);
    }
    // gate weights of this wave's 32 channels: B fragments of the 16 K steps (lane half kh
    // supplies inputs 16 s + 8 kh .. + 7 of step s)
    const int ln = lane & 31, kh = lane >> 5;
    bf16x8 wA[kBs / 16], wX[kBs / 16];
    {
        const size_t chn = (size_t)head * kBs + 32 * wv + ln;
        const uint16_t* war = static_cast<const uint16_t*>(a.wa) + chn * kBs;
        const uint16_t* wxr = static_cast<const uint16_t*>(a.wx) + chn * kBs;
#pragma unroll
        for (int s = 0; s < kBs / 16; ++s) {
            wA[s] = *reinterpret_cast<const bf16x8*>(war + 16 * s + 8 * kh);
            wX[s] = *reinterpret_cast<const bf16x8*>(wxr + 16 * s + 8 * kh);
        }
    }
    __syncthreads();  // tables

    const int pw = wv & 1, tg = wv >> 1;      // conv tile: channels 128 pw .., tokens 16 tg ..
    const int xw0 = wv * kFXElems, yw0 = wv * kFYElems;
    const int cw0 = 32 * wv;                  // output channels of this wave
    // A-fragment row -> token: lane ln supplies token 32 ((ln >> 2) & 1) + 4 (ln >> 3) + (ln & 3)
    // (+ 16 for tile 1), so result register j of lane (kh, ln) is token 32 kh + j (+ 16)
    const int atok = 32 * ((ln >> 2) & 1) + 4 * (ln >> 3) + (ln & 3);
    const int rowb = D * 2;

    // copies of unit un into this wave's LDS regions: x rows (with the 3-token halo: the
    // previous tokens, the conv0 window or zeros), and y and dout rows of its 32 channels
    auto copy_x = [&](int un) {
        const int b = un / nseg, t0 = (un % nseg) * kFSeg;
        const __amdgpu_buffer_rsrc_t rx = rsrc_at(static_cast<const uint16_t*>(a.x) + (size_t)b * T * D);
        const int coff = (head * kBs + 128 * pw + 8 * (lane & 15)) * 2;
        const int tok0 = t0 + 16 * tg - 3 + (lane >> 4);
        if (t0 == 0 && tg == 0) {
            // rows 0..2 of the first copy are tokens -3..-1: the conv0 window (a resource of
            // length 0 reads zeros when there is none); built from a wave-uniform pointer
            const uint64_t cp = reinterpret_cast<uint64_t>(a.conv0 ? a.conv0 : a.x);
            const uint32_t c_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(cp >> 32));
            const uint32_t c_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)cp);
            const __amdgpu_buffer_rsrc_t rc = rsrc_len(
                reinterpret_cast<void*>(((uint64_t)c_hi << 32) | (uint64_t)c_lo), a.conv0 ? 0xffffffffu : 0u);
            if ((lane >> 4) == 3) __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, x_lds + xw0, 16, coff, 0, 0, 0);
            else __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, x_lds + xw0, 16, ((b * 3 + (lane >> 4)) * D) * 2 + coff, 0, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, x_lds + xw0, 16, min(tok0, T - 1) * rowb + coff, 0, 0, 0);
        }
#pragma unroll
        for (int q = 1; q < 5; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, x_lds + xw0 + q * 512, 16,
                                                     min(tok0 + 4 * q, T - 1) * rowb + coff, 0, 0, 0);
    };
    // eight copies (wait counts below rely on that number)
    auto copy_yd = [&](int un) {
        const int b = un / nseg, t0 = (un % nseg) * kFSeg;
        const size_t tmo = (size_t)b * T * D + (size_t)head * kBs + cw0;
        const __amdgpu_buffer_rsrc_t ry = rsrc_at(static_cast<const uint16_t*>(a.y) + tmo);
        const __amdgpu_buffer_rsrc_t rd = rsrc_at(static_cast<const uint16_t*>(a.dout) + tmo);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int off = min(t0 + 16 * q + (lane >> 2), T - 1) * rowb + 16 * (lane & 3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, y_lds + yw0 + f_yrow(16 * q), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, d_lds + yw0 + f_yrow(16 * q), 16, off, 0, 0, 0);
        }
    };
    // this lane's conv taps and biases (channels 128 pw + 2 lane, + 1), the same for every unit
    const float4 tl = ctap[128 * pw + 2 * lane], th = ctap[128 * pw + 2 * lane + 1];
    const float bl = cbias[128 * pw + 2 * lane], bh = cbias[128 * pw + 2 * lane + 1];
    if (jw < units) {
        copy_x(jw);
        copy_yd(jw);
    }

    // A unit's copies go out a unit ahead: x right after the last unit's conv has read the x
    // rows, y and dout right after the last unit's aggregate walk has read those.  The wait at
    // the top of a unit needs only x: the eight y/dout copies are the youngest memory operations
    // in flight and loads complete in order, so vmcnt(8) leaves exactly them outstanding (and
    // waits for the last unit's stores).  y and dout are waited for before the walk, a conv and
    // an MFMA phase after they were issued.
    for (int un = jw; un < units; un += wph) {
        const int b = un / nseg, seg = un % nseg;
        const int t0 = seg * kFSeg, nt = min(kFSeg, T - t0);
        const size_t m0 = (size_t)b * T + t0;
        const bool more = un + wph < units;

        __builtin_amdgcn_s_waitcnt(0x0f78);   // vmcnt(8): this wave's x rows of this unit have landed
        f_lds_barrier();   // every wave's x rows; every wave's reads of the last unit's u tile done

        // ---- 2. conv: lane = channel pair 128 pw + 2 lane, tokens 16 tg .. 16 tg + 15 ----
        {
            const int c = 128 * pw + 2 * lane;
            const int ixr = f_opaque(xw0 / 2 + lane);
            const int iuw = f_opaque(c / 2);
            uint32_t xr[19];
#pragma unroll
            for (int r = 0; r < 19; ++r) xr[r] = x_lds32[ixr + r * 64];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                float lo = __builtin_fmaf(tl.x, bf_lo(xr[k]), bl);
                lo = __builtin_fmaf(tl.y, bf_lo(xr[k + 1]), lo);
                lo = __builtin_fmaf(tl.z, bf_lo(xr[k + 2]), lo);
                lo = __builtin_fmaf(tl.w, bf_lo(xr[k + 3]), lo);
                float hi = __builtin_fmaf(th.x, bf_hi(xr[k]), bh);
                hi = __builtin_fmaf(th.y, bf_hi(xr[k + 1]), hi);
                hi = __builtin_fmaf(th.z, bf_hi(xr[k + 2]), hi);
                hi = __builtin_fmaf(th.w, bf_hi(xr[k + 3]), hi);
                const uint32_t pk = pack2bf(lo, hi);
                const int tt = 16 * tg + k;   // wave-uniform
                u_lds32[iuw + f_urow(tt) * (kFRow / 2)] = pk;
            }
        }
        f_lds_barrier();   // u tile complete; this wave's x rows are read
        {
            // U out of the tile: 64 rows of 512 bytes as 16-byte stores, four per thread
            // (rows past the unit's tokens fall outside the resource and are dropped)
            const __amdgpu_buffer_rsrc_t ru = rsrc_len(w.U + ((size_t)head * M + m0) * kBs, (uint32_t)nt * kBs * 2);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int id = q * kFThreads + tid, row = id >> 5, ch = id & 31;
                const uint4 v = *reinterpret_cast<const uint4*>(u_lds + f_urow(row) * kFRow + 8 * ch);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), ru, (row * kBs + 8 * ch) * 2, 0, 0);
            }
        }
        if (more) copy_x(un + wph);

        // ---- 3. gate pre-activations ----
        f32x16 accA[2], accX[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) { accA[0][e] = 0.0f; accX[0][e] = 0.0f; accA[1][e] = 0.0f; accX[1][e] = 0.0f; }
        {   // tile 0 here; tile 1's MFMAs run beside tile 0's walk below
            const int ia = f_opaque(f_urow(atok) * kFRow + 8 * kh);
#pragma unroll
            for (int s = 0; s < kBs / 16; ++s) {
                const bf16x8 A = *reinterpret_cast<const bf16x8*>(u_lds + ia + 16 * s);
                accA[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wA[s], accA[0], 0, 0, 0);
                accX[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wX[s], accX[0], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);  // one fragment in flight: the weights hold half the registers
            }
        }

        // ---- 4. R, I out; chunk aggregates of chunk 2 seg + kh over its 32 tokens ----
        // this wave's y and dout rows of this unit: younger than them are this unit's U stores
        // and, when there is a next unit, its five or six x copies, which cannot land before
        // them; vmcnt(5) therefore implies they have landed (and leaves the x copies in flight)
        if (more) __builtin_amdgcn_s_waitcnt(0x0f75);   // vmcnt(5)
        else f_wait_vmem();
        {
            const int c = cw0 + ln;
            const float bA = gba[c], bX = gbx[c], lsg = glsg[c];
            const size_t hb = ((size_t)head * M + m0) * kBs;
            const __amdgpu_buffer_rsrc_t rr = rsrc_len(w.R + hb, (uint32_t)nt * kBs * 2);
            const __amdgpu_buffer_rsrc_t ri = rsrc_len(w.I + hb, (uint32_t)nt * kBs * 2);
            // token tt = 32 kh + 16 mt + j: u at row
            // f_urow(tt) = 32 kh + 16 mt + j + kh (12 - 8 (j / 4)) (bits 2..3 of j flipped for kh = 1);
            // y and dout at yb + (16 mt + j) * 32
            int iub[4];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) iub[g4] = f_opaque((32 * kh + kh * (12 - 8 * g4)) * kFRow + c);
            const int yb = f_opaque(yw0 + f_yrow(32 * kh) + ln);
            const int ia1 = f_opaque(f_urow(atok + 16) * kFRow + 8 * kh);
            float A = 1.0f, Bh = 0.0f, Q = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (mt == 0) {   // K step j of tile 1
                        const bf16x8 Af = *reinterpret_cast<const bf16x8*>(u_lds + ia1 + 16 * j);
                        accA[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Af, wA[j], accA[1], 0, 0, 0);
                        accX[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Af, wX[j], accX[1], 0, 0, 0);
                    }
                    const int tj = 16 * mt + j;
                    const uint16_t r16 = f2bf(accA[mt][j] + bA), i16 = f2bf(accX[mt][j] + bX);
                    const Gate g = gate_of(bf2f(r16), bf2f(i16), lsg);
                    const float u = bf2f(u_lds[iub[j >> 2] + tj * kFRow]);
                    A *= g.a;
                    Bh = __builtin_fmaf(g.a, Bh, g.m * g.i * u);
                    const float yv = bf2f(y_lds[yb + tj * 32]);
                    const float dov = bf2f(d_lds[yb + tj * 32]);
                    Q = __builtin_fmaf(A, dov * gelu_and_grad(yv).x, Q);
                    // R and I of this token take the places of its y and dout, just read
                    y_lds[yb + tj * 32] = r16;
                    d_lds[yb + tj * 32] = i16;
                    __builtin_amdgcn_sched_barrier(0);  // bound the loads hoisted ahead
                }
            }
            // [B * nch][D] rows of this unit's chunks; a unit of 32 tokens has no second chunk,
            // and the resource's range drops its stores (unconditional stores: a branch here
            // would let the compiler sink the whole gate computation below all the R/I stores)
            const size_t row0 = ((size_t)b * nch + t0 / kChunk) * D;
            const uint32_t nb = (uint32_t)(nt / kChunk) * (uint32_t)D * 4;
            const int vo = f_opaque((kh * D + head * kBs + c) * 4);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(A), rsrc_len(w.aggA + row0, nb), vo, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Bh), rsrc_len(w.aggB + row0, nb), vo, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Q), rsrc_len(w.bQ + row0, nb), vo, 0, 0);
            // R and I out of the y and dout regions: 64 rows of this wave's 32 channels, four
            // lanes per 64-byte row, 16-byte stores (rows past the unit's tokens are dropped)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = 16 * q + (lane >> 2), ch = lane & 3;
                const int li = yw0 + f_yrow(16 * q) + (lane >> 2) * 32 + 8 * ch;
                const uint4 vr = *reinterpret_cast<const uint4*>(y_lds + li);
                const uint4 vi = *reinterpret_cast<const uint4*>(d_lds + li);
                const int off = (row * kBs + cw0 + 8 * ch) * 2;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, vr), rr, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, vi), ri, off, 0, 0);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's reads of its y and dout regions are done
        if (more) copy_yd(un + wph);
    }
    f_wait_vmem();
}

// ---- carries over the chunks: h entering each chunk (forward) and c entering it from the
// right (reverse); the reverse carry past the first chunk is dh0.  Two levels: each group of
// kGroupChunks chunks is composed into one (A, B) and (A, Q) pair, the groups are walked in
// sequence per (sequence, channel), then each group hands its entry carries to its chunks.
// Every step is the same fma in the same order as a plain walk over the chunks would take
// within a group, and composed pairs across groups. -----------------------------------------
__global__ void __launch_bounds__(256) bwd_carry_group_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk, ng = groups_of(nch);
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;   // (b, group, d)
    if (idx >= (size_t)a.B * ng * a.D) return;
    const int d = (int)(idx % a.D), gi = (int)((idx / a.D) % ng), b = (int)(idx / ((size_t)ng * a.D));
    const int c0 = gi * kGroupChunks, c1 = min(nch, c0 + kGroupChunks);
    // forward: h_out = A h_in + Bf; reverse: c_out (entering the group's first chunk from the
    // right) = A c_in + Q, with A the product of the chunks' A
    float A = 1.0f, Bf = 0.0f;
    for (int c = c0; c < c1; ++c) {
        const size_t e = ((size_t)b * nch + c) * a.D + d;
        A *= w.aggA[e];
        Bf = __builtin_fmaf(w.aggA[e], Bf, w.aggB[e]);
    }
    float Q = 0.0f;
    for (int c = c1 - 1; c >= c0; --c) {
        const size_t e = ((size_t)b * nch + c) * a.D + d;
        Q = __builtin_fmaf(w.aggA[e], Q, w.bQ[e]);
    }
    w.sA[idx] = A;
    w.sB[idx] = Bf;
    w.sQ[idx] = Q;
}

__global__ void __launch_bounds__(256) bwd_carry_walk_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk, ng = groups_of(nch);
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;   // (b, d)
    if (idx >= (size_t)a.B * a.D) return;
    const int d = (int)(idx % a.D), b = (int)(idx / a.D);
    float h = a.h0 ? a.h0[idx] : 0.0f;
    for (int gi = 0; gi < ng; ++gi) {
        const size_t e = ((size_t)b * ng + gi) * a.D + d;
        w.sh[e] = h;
        h = __builtin_fmaf(w.sA[e], h, w.sB[e]);
    }
    float cc = a.dh_last ? a.dh_last[idx] : 0.0f;
    for (int gi = ng - 1; gi >= 0; --gi) {
        const size_t e = ((size_t)b * ng + gi) * a.D + d;
        w.sc[e] = cc;
        cc = __builtin_fmaf(w.sA[e], cc, w.sQ[e]);
    }
    a.dh0[idx] = cc;
}

__global__ void __launch_bounds__(256) bwd_carry_fill_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk, ng = groups_of(nch);
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;   // (b, group, d)
    if (idx >= (size_t)a.B * ng * a.D) return;
    const int d = (int)(idx % a.D), gi = (int)((idx / a.D) % ng), b = (int)(idx / ((size_t)ng * a.D));
    const int c0 = gi * kGroupChunks, c1 = min(nch, c0 + kGroupChunks);
    float h = w.sh[idx];
    for (int c = c0; c < c1; ++c) {
        const size_t e = ((size_t)b * nch + c) * a.D + d;
        w.carry[e] = h;
        h = __builtin_fmaf(w.aggA[e], h, w.aggB[e]);
    }
    float cc = w.sc[idx];
    for (int c = c1 - 1; c >= c0; --c) {
        const size_t e = ((size_t)b * nch + c) * a.D + d;
        w.cin[e] = cc;
        cc = __builtin_fmaf(w.aggA[e], cc, w.bQ[e]);
    }
}

// ---- per-element gradients of one chunk ----------------------------------------------------
// The block's inputs (32 tokens x 256 channels of R, I, U, y and dout: 80 KB) come into LDS by
// bulk global -> LDS copies, 1 KB per instruction, all in flight at once; each lane then walks
// its channel out of LDS (with per-token global loads the pass waited on memory latency).  The
// gradients of the gate pre-activations and of y replace R, I and y in LDS as the backward walk
// consumes them, and leave as whole rows at the end: dRI head-major and dy token-major in
// coalesced 16-byte chunks.
__global__ void __launch_bounds__(128, 2) bwd_grad_kernel(BwdArgs a, BwdBufs w) {
    constexpr int kHalf = kBs / 2;   // channels per block: half a head
    __shared__ __attribute__((aligned(16))) uint16_t tR[kChunk * kHalf], tI[kChunk * kHalf],
        tU[kChunk * kHalf], tY[kChunk * kHalf], tD[kChunk * kHalf];
    // blockIdx = ((b * nch + c) * H + h) * 2 + half
    const int nch = a.T / kChunk;
    const int half = (int)(blockIdx.x & 1u);
    const unsigned bh = blockIdx.x >> 1;
    const int h = (int)(bh % (unsigned)a.H);
    const unsigned bc = bh / (unsigned)a.H;
    const int c_ = (int)(bc % (unsigned)nch), b_ = (int)(bc / (unsigned)nch);
    const size_t m0 = (size_t)b_ * a.T + (size_t)c_ * kChunk;
    const int t = threadIdx.x, k = half * kHalf + t, d = h * kBs + k;
    const int wv = t >> 6, lane = t & 63;
    const size_t idx = (size_t)blockIdx.x * kHalf + t;   // ((b * nch + c) * D + d)
    const size_t M = (size_t)a.B * a.T;
    const size_t hmo = ((size_t)h * M + m0) * kBs;   // head-major element of token m0
    const size_t tmo = m0 * a.D + (size_t)h * kBs;   // token-major element of token m0
    {
        const auto rR = rsrc_at(w.R + hmo), rI = rsrc_at(w.I + hmo), rU = rsrc_at(w.U + hmo);
        const auto rY = rsrc_at(static_cast<const uint16_t*>(a.y) + tmo);
        const auto rDo = rsrc_at(static_cast<const uint16_t*>(a.dout) + tmo);
        const int sD = 2 * a.D;
        // 1 KB chunk c of a tile is its rows 4c .. 4c+3 (256 bytes each: this half's channels)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * wv + j, row = 4 * c + (lane >> 4), col = half * 256 + (lane & 15) * 16;
            const int ho = row * (2 * kBs) + col, to = row * sD + col;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rR, tR + c * 512, 16, ho, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rI, tI + c * 512, 16, ho, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rU, tU + c * 512, 16, ho, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rY, tY + c * 512, 16, to, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rDo, tD + c * 512, 16, to, 0, 0, 0);
        }
    }
    const float lsg = log_sigmoid(a.lambda[d]);
    const float sg = expf(lsg);
    // per channel: log a = c2 r; log2 a = c2l r; d/dLambda log a = c1 r
    const float c2 = 8.0f * lsg, c2l = c2 * kLog2e, c2x2 = 2.0f * c2, c1 = 8.0f * (1.0f - sg);
    float hv = w.carry[idx];
    float cc = w.cin[idx];
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's copies have landed
    __syncthreads();                      // and the other wave's
    // the forward re-run keeps h_{t-1}, a and sqrt(1 - a^2) of each token for the walk (the
    // registers are free: LDS allows two waves per SIMD); the walk re-forms only r and i, and
    // h_t is the re-run's next h_{t-1}
    float hp[kChunk], ca[kChunk], cm[kChunk], cr[kChunk], ci[kChunk];
#pragma unroll
    for (int tt = 0; tt < kChunk; ++tt) {
        hp[tt] = hv;
        const int e = tt * kHalf + t;
        const float r = sigm(bf2f(tR[e])), i = sigm(bf2f(tI[e]));
        const float av = __builtin_amdgcn_exp2f(r * c2l);
        const float m = sqrt_one_minus_a2(r * c2x2, av);
        ca[tt] = av;
        cm[tt] = m;
        cr[tt] = r;
        ci[tt] = i;
        hv = __builtin_fmaf(av, hv, m * i * bf2f(tU[e]));
    }
    const auto rDuv = rsrc_at(w.duv + hmo);
    float slam = 0.0f, sba = 0.0f, sbx = 0.0f;
#pragma unroll
    for (int tt = kChunk - 1; tt >= 0; --tt) {
        const int e = tt * kHalf + t;
        const float u = bf2f(tU[e]);
        const float r = cr[tt], i = ci[tt];
        const float av = ca[tt], m = cm[tt];
        const float ht = tt + 1 < kChunk ? hp[tt + 1] : hv;
        const float yv = bf2f(tY[e]), dov = bf2f(tD[e]);
        const float2 gg = gelu_and_grad(yv);
        const float dh = __builtin_fmaf(dov, gg.x, cc);
        tY[e] = f2bf(dov * ht * gg.y);
        const float dv = dh * (m * i);
        st_f32(rDuv, 4 * k, tt * 4 * kBs, dv);
        // q = a dL/da with m = sqrt(1 - a^2): a (h_{t-1} dh - dh i u a / m), and since
        // a h_{t-1} = h_t - m i u and a^2 / m = 1 / m - m, q = dh (h_t - i u / m)
        const float q = dh * (ht - (i * u) * __builtin_amdgcn_rcpf(m));
        const float qr = q * r;
        slam = __builtin_fmaf(qr, c1, slam);
        const float dRp = (qr * c2) * (1.0f - r), dIp = (dv * u) * (1.0f - i);
        sba += dRp;
        sbx += dIp;
        tR[e] = f2bf(dRp);
        tI[e] = f2bf(dIp);
        cc = dh * av;
    }
    w.plam[idx] = slam;
    w.pba[idx] = sba;
    w.pbx[idx] = sbx;
    __syncthreads();   // every lane's column of dR, dI and dy is in LDS
    {
        // dRI, head-major: token tt's row is [dR (256) | dI (256)]; this block's part of it is
        // bytes half * 256 .. + 255 of each half.  16-byte chunk c: token c / 32, then dR or dI
        // ((c / 16) & 1) and chunk c % 16 of this half.
        uint16_t* const dri = w.dRI + 2 * hmo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = t + 128 * i, tt = c >> 5, which = (c >> 4) & 1, q = c & 15;
            const uint16_t* src = (which ? tI : tR) + tt * kHalf + 8 * q;
            *reinterpret_cast<uint4*>(dri + (size_t)tt * 2 * kBs + which * kBs + half * kHalf + 8 * q) =
                *reinterpret_cast<const uint4*>(src);
        }
        // dy, token-major: 16-byte chunk c is token c / 16, chunk c % 16 of this half
        uint16_t* const dyb = static_cast<uint16_t*>(a.dy) + tmo + half * kHalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 128 * i, tt = c >> 4, q = c & 15;
            *reinterpret_cast<uint4*>(dyb + (size_t)tt * a.D + 8 * q) =
                *reinterpret_cast<const uint4*>(tY + tt * kHalf + 8 * q);
        }
    }
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
    const size_t pe = ((size_t)b * nch + c) * a.D + d, nc = (size_t)a.B * nch * a.D;
#pragma unroll
    for (int j = 0; j < 5; ++j) {   // [5][B * nch * D]: eight consecutive channels per store pair
        float v8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v8[q] = j < 4 ? sw[q][j] : sb[q];
        float4* pc = reinterpret_cast<float4*>(w.pconv + j * nc + pe);
        pc[0] = make_float4(v8[0], v8[1], v8[2], v8[3]);
        pc[1] = make_float4(v8[4], v8[5], v8[6], v8[7]);
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

// ---- gradient of u through both gates: dU_h = [dR | dI]_h [W_a[h]^T | W_x[h]^T]^T, K = 512 ----
// One workgroup of eight waves per CU pinned to a head: wave w keeps the B fragments of
// [W_a^T | W_x^T] for u channels 32w .. 32w + 31 (all 512 K) in VGPRs, and the workgroup walks
// 64-token units of dRI rows, double-buffered in LDS (one 1 KB row per copy, 16 bytes of padding
// per row so that an A fragment's 32 rows fall on different banks).  K runs in natural order in
// steps of 16 and the result is rounded as the projection GEMM's epilogue rounds it, so dU is
// the same as that GEMM's.  The bf16 tile is staged in the unit's stage and leaves as 16-byte
// stores one unit later (held in registers), so the wait for the next copies never includes
// stores issued just before it.
constexpr int kDgRow = 4 * kBs + 16;            // bytes of one staged dRI row (512 bf16 + padding)
constexpr int kDgStage = kFSeg * kDgRow;
__device__ __forceinline__ int dg_orow(int r) { return r * 2 * kBs + ((r >> 5) << 6); }  // output row, bytes

__global__ void __launch_bounds__(kFThreads) bwd_dgate_kernel(BwdArgs a, BwdBufs w, int wph) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kDgStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned G = gridDim.x, bid = blockIdx.x;
    const unsigned xcd = bid & 7u, jx = bid >> 3, per = G >> 3, rem = G & 7u;
    const unsigned slot = xcd * per + min(xcd, rem) + jx;
    const int head = (int)(slot / (unsigned)wph), jw = (int)(slot % (unsigned)wph);
    if (head >= a.H) return;
    const int B = a.B, T = a.T;
    const size_t M = (size_t)B * T;
    const int nseg = (T + kFSeg - 1) / kFSeg, units = B * nseg;
    const int ln = lane & 31, kh = lane >> 5;
    bf16x8 wB[2 * kBs / 16];
    {
        const uint16_t* wr = w.Wt + ((size_t)head * kBs + 32 * wv + ln) * 2 * kBs;
#pragma unroll
        for (int s2 = 0; s2 < 2 * kBs / 16; ++s2) wB[s2] = *reinterpret_cast<const bf16x8*>(wr + 16 * s2 + 8 * kh);
    }
    const int atok = 32 * ((ln >> 2) & 1) + 4 * (ln >> 3) + (ln & 3);
    // rows 8 wv .. 8 wv + 7 of unit un into stage st (rows past the unit repeat its last row)
    auto copy_rows = [&](int un, int st) {
        const int b = un / nseg, t0 = (un % nseg) * kFSeg, nt = min(kFSeg, T - t0);
        const __amdgpu_buffer_rsrc_t rs = rsrc_at(w.dRI + ((size_t)head * M + (size_t)b * T + t0) * 2 * kBs);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 8 * wv + q;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds + st * kDgStage + r * kDgRow, 16,
                                                     min(r, nt - 1) * 4 * kBs + 16 * lane, 0, 0, 0);
        }
    };
    uint4 sv[4];                 // the last unit's staged output, stored one unit late
    size_t pm0 = 0;
    int pnt = 0;
    bool pending = false;
    auto store_prev = [&]() {
        const __amdgpu_buffer_rsrc_t ro = rsrc_len(w.dUg + ((size_t)head * M + pm0) * kBs, (uint32_t)pnt * kBs * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int id = q * kFThreads + tid, row = id >> 5, ch = id & 31;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, sv[q]), ro, (row * kBs + 8 * ch) * 2, 0, 0);
        }
    };
    if (jw < units) copy_rows(jw, 0);
    int st = 0;
    for (int un = jw; un < units; un += wph, st ^= 1) {
        const int b = un / nseg, t0 = (un % nseg) * kFSeg;
        f_wait_vmem();     // this wave's rows of this unit (and the stores issued a unit ago)
        f_lds_barrier();   // every wave's rows; every wave's reads of the other stage are done
        if (un + wph < units) copy_rows(un + wph, st ^ 1);
        if (pending) store_prev();
        const unsigned char* const sa = lds + st * kDgStage;
        f32x16 acc0, acc1;
#pragma unroll
        for (int e = 0; e < 16; ++e) { acc0[e] = 0.0f; acc1[e] = 0.0f; }
        const int ia0 = f_opaque(atok * kDgRow + 16 * kh), ia1 = f_opaque((atok + 16) * kDgRow + 16 * kh);
#pragma unroll
        for (int s2 = 0; s2 < 2 * kBs / 16; ++s2) {
            const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(sa + ia0 + 32 * s2);
            const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(sa + ia1 + 32 * s2);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, wB[s2], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, wB[s2], acc1, 0, 0, 0);
        }
        f_lds_barrier();   // every wave's reads of this stage are done: it takes the output now
        unsigned char* const so = lds + st * kDgStage;
        {
            // token 32 kh + 16 mt + j, channel 32 wv + ln; + 0.0f as the GEMM's epilogue adds a
            // zero bias (a -0 sum leaves as +0)
            const int ob = f_opaque(dg_orow(32 * kh) + 2 * (32 * wv + ln));
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                *reinterpret_cast<uint16_t*>(so + ob + j * 2 * kBs) = f2bf(acc0[j] + 0.0f);
                *reinterpret_cast<uint16_t*>(so + ob + (16 + j) * 2 * kBs) = f2bf(acc1[j] + 0.0f);
            }
        }
        f_lds_barrier();   // the output tile is complete
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int id = q * kFThreads + tid, row = id >> 5, ch = id & 31;
            sv[q] = *reinterpret_cast<const uint4*>(so + dg_orow(row) + 16 * ch);
        }
        pm0 = (size_t)b * T + t0;
        pnt = min(kFSeg, T - t0);
        pending = true;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (pending) store_prev();
    f_wait_vmem();
}

// ---- gate weight gradients from the head-major dRI and U: [dW_a; dW_x]_h = [dR | dI]_h^T U_h ----
// K runs over tokens, which are the rows (not the contiguous dimension) of both operands, so the
// MFMA fragments (eight consecutive K per lane) are gathered from LDS with 2-byte reads.  One
// workgroup (four waves of 128 x 128) per 256 x 256 output tile (head h, dR or dI rows) and
// token range; 32-token steps through two LDS stages filled by buffer loads (1 KB = two 512-byte
// rows per copy; 16 bytes of padding after every two rows put the two half-waves' reads, eight
// rows apart, on different banks).  The fp32 tile of each range goes to wpart and the ranges are
// summed in order by bwd_wgrad_sum_kernel (bitwise repeatable).
constexpr int kWgRowB = 2 * kBs;             // bytes of one staged row (256 bf16)
constexpr int kWgBlk = 2 * kWgRowB + 16;     // one copy: two rows and the padding
constexpr int kWgTile = 16 * kWgBlk;         // 32 rows
constexpr int kWgStage = 2 * kWgTile;        // dRI and U rows of one step

__device__ __forceinline__ bf16x8 wg_frag(const unsigned char* tile, int r0, int col) {
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int r = r0 + e;
        v[e] = *reinterpret_cast<const unsigned short*>(tile + (r >> 1) * kWgBlk + (r & 1) * kWgRowB + 2 * col);
    }
    return __builtin_bit_cast(bf16x8, v);
}

__global__ void __launch_bounds__(256, 1) bwd_wgrad_kernel(BwdArgs a, BwdBufs w) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kWgStage];
    const int H = a.H, S = w.wsplits;
    const unsigned bid = blockIdx.x;     // (s * H + h) * 2 + ohalf
    const int ohalf = (int)(bid & 1u), h = (int)((bid >> 1) % (unsigned)H), s = (int)((bid >> 1) / (unsigned)H);
    const size_t M = (size_t)a.B * a.T;
    const int KS = (int)(M / 32);
    const int k0 = (int)((long long)KS * s / S), k1 = (int)((long long)KS * (s + 1) / S);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const uint16_t* const abase = w.dRI + (size_t)h * M * 2 * kBs + ohalf * kBs;   // row m at + m * 512
    const uint16_t* const bbase = w.U + (size_t)h * M * kBs;                       // row m at + m * 256
    // copies of step ks into stage st: this wave's blocks 4 wv .. 4 wv + 3 of each tile
    auto issue = [&](int ks, int st) {
        const size_t m0 = (size_t)ks * 32;
        const __amdgpu_buffer_rsrc_t ra = rsrc_at(abase + m0 * 2 * kBs), rb = rsrc_at(bbase + m0 * kBs);
        unsigned char* const sa = lds + st * kWgStage;
        const int row = lane >> 5, colb = (lane & 31) * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int blk = 4 * wv + q;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, sa + blk * kWgBlk, 16, (2 * blk + row) * (4 * kBs) + colb, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, sa + kWgTile + blk * kWgBlk, 16, (2 * blk + row) * (2 * kBs) + colb, 0, 0, 0);
        }
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if (k0 < k1) issue(k0, 0);
    for (int ks = k0; ks < k1; ++ks) {
        const int st = (ks - k0) & 1;
        if (ks + 1 < k1) {
            issue(ks + 1, st ^ 1);   // that stage's reads ended at the last step's final barrier
            __builtin_amdgcn_s_waitcnt(0x0f78);   // vmcnt(8): this step's eight copies have landed
        } else {
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        }
        f_lds_barrier();   // every wave's copies of this step (each waited for its own above)
        const unsigned char* const sa = lds + st * kWgStage;
        const unsigned char* const sb = sa + kWgTile;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int r0 = 16 * sub + 8 * (lane >> 5);   // K slice of this lane: tokens r0 .. r0 + 7
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = wg_frag(sa, r0, 128 * wm + 32 * i + (lane & 31));
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = wg_frag(sb, r0, 128 * wn + 32 * j + (lane & 31));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        f_lds_barrier();   // this stage is no longer read (the next step refills it)
    }
    // tile element (o, c): block (i, j) register e holds o = 128 wm + 32 i + 8 (e / 4) + 4 (lane / 32)
    // + e % 4 and c = 128 wn + 32 j + lane % 32
    float* const out = w.wpart + (((size_t)s * H + h) * 2 * kBs + (size_t)ohalf * kBs) * kBs;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int o = 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int c = 128 * wn + 32 * j + (lane & 31);
                out[(size_t)o * kBs + c] = acc[i][j][e];
            }
}

// dW_a, dW_x = the token ranges' partial tiles added in range order
__global__ void __launch_bounds__(256) bwd_wgrad_sum_kernel(BwdArgs a, BwdBufs w) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;   // (h, o in 0..511, c)
    const size_t per = (size_t)2 * kBs * kBs;
    if (idx >= (size_t)a.H * per) return;
    const size_t h = idx / per, r = idx % per;
    float v = 0.0f;
    for (int s = 0; s < w.wsplits; ++s) v += w.wpart[((size_t)s * a.H + h) * per + r];
    if (r < (size_t)kBs * kBs) a.dwa[h * kBs * kBs + r] = v;
    else a.dwx[h * kBs * kBs + (r - (size_t)kBs * kBs)] = v;
}

// Fixed-order sums of the per-chunk partials, in two passes with consecutive lanes on
// consecutive channels (whole-row loads): pass 1 sums each of kRedParts consecutive ranges of
// the B * nch partials in order, pass 2 adds the ranges in order.
__global__ void __launch_bounds__(256) bwd_reduce_part_kernel(BwdArgs a, BwdBufs w) {
    const int nch = a.T / kChunk, np = a.B * nch;
    const int d = blockIdx.x * 256 + threadIdx.x, r = blockIdx.y;
    if (d >= a.D) return;
    const int per = (np + kRedParts - 1) / kRedParts, q0 = r * per, q1 = min(np, q0 + per);
    const size_t nc = (size_t)np * a.D;
    float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int q = q0; q < q1; ++q) {
        const size_t e = (size_t)q * a.D + d;
        v[0] += w.plam[e];
        v[1] += w.pba[e];
        v[2] += w.pbx[e];
#pragma unroll
        for (int j = 0; j < 5; ++j) v[3 + j] += w.pconv[j * nc + e];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) w.red[((size_t)r * 8 + j) * a.D + d] = v[j];
}

__global__ void __launch_bounds__(256) bwd_reduce_kernel(BwdArgs a, BwdBufs w) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= a.D) return;
    float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int r = 0; r < kRedParts; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] += w.red[((size_t)r * 8 + j) * a.D + d];
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
    RG_LAUNCH(bwd_wtrans_kernel, (size_t)a.H * kBs * 2 * kBs);
    {   // U, the gate pre-activations R and I, and the chunk aggregates: one persistent launch
        const int wph = std::max(1, device_cu_count() / a.H);
        hipLaunchKernelGGL(bwd_front_kernel, dim3((unsigned)(wph * a.H)), dim3(kFThreads), 0, s, a, w, wph);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        const size_t ngl = (size_t)a.B * groups_of((int)nch) * a.D;
        RG_LAUNCH(bwd_carry_group_kernel, ngl);
        RG_LAUNCH(bwd_carry_walk_kernel, (size_t)a.B * a.D);
        RG_LAUNCH(bwd_carry_fill_kernel, ngl);
    }
    hipLaunchKernelGGL(bwd_grad_kernel, dim3((unsigned)(nlane / (kBs / 2))), dim3(kBs / 2), 0, s, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {   // gradient of u through the gates: one persistent launch, the weights held in registers
        const int wph = std::max(1, device_cu_count() / a.H);
        hipLaunchKernelGGL(bwd_dgate_kernel, dim3((unsigned)(wph * a.H)), dim3(kFThreads), 0, s, a, w, wph);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // gate weight gradients (K = B * T), all heads in one launch, then the ranges' sum
    hipLaunchKernelGGL(bwd_wgrad_kernel, dim3((unsigned)(w.wsplits * a.H * 2)), dim3(256), 0, s, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    RG_LAUNCH(bwd_wgrad_sum_kernel, (size_t)a.H * 2 * kBs * kBs);
    RG_LAUNCH(bwd_conv_kernel, nlane / 8);
    hipLaunchKernelGGL(bwd_reduce_part_kernel, dim3((unsigned)((a.D + 255) / 256), kRedParts),
                       dim3(256), 0, s, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((a.D + 255) / 256)), dim3(256), 0, s, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
#undef RG_LAUNCH
    return hipSuccess;
}

}  // namespace rglru
