// Local sliding-window multi-query attention, for gfx950 (CDNA4): the model's other
// temporal-mixing block.  The page "Gemma 詳解：RecurrentGemma 架構" (section "含區域 MQA 的殘差
// 區塊" and the printout's RecurrentGemmaSdpaAttention) gives Hq query heads of dh = 256
// sharing one key/value head (multi-query attention), rotary position embedding on q and k
// following the base Gemma model, and attention restricted to a fixed window of past tokens
// (section "區域注意力視窗大小": 2k).  Here query t attends to tokens t - W + 1 .. t:
//
//   o[t, h] = sum_s softmax_s(q[t, h] . k[s] / sqrt(dh)) v[s]
//
// after RoPE turns each pair (x_i, x_{i + dh/2}) of q and k by t * base^(-2 i / dh).
//
// Prefill, two kernels (decode, with a ring KV cache, is further down):
//   attn_prep_kernel  RoPE on q and k (angles in fp64), and v regrouped in fours of keys,
//                     [B][T/4][dh][4], the order in which the P.V MFMA reads it;
//   attn_fwd_kernel   one workgroup per (sequence, head, 128 queries); each wave holds 32
//                     queries.  Scores are formed transposed, S^T = K Q^T (keys x queries), so a
//                     lane owns one query: the softmax runs within the lane (and its partner
//                     lane, which holds the query's other 16 keys).  The v_mfma_f32_32x32x16_bf16
//                     result puts keys 8 g + 4 (l / 32) + i in register 4 g + i; taking registers
//                     8 k .. 8 k + 7 as the K slice of the next MFMA, the probabilities feed
//                     O^T += V^T P^T straight from registers, with V read as two groups of four
//                     keys per lane.  Keys arrive in tiles of 32 (K 16 KB, V 16 KB) through two
//                     LDS stages, copied by LDS-DMA one tile ahead.  The online softmax
//                     keeps a reference maximum per query and rescales the output only when a
//                     tile's maximum exceeds it by 2^8 (in exp2 units); the normaliser uses the
//                     same reference, so the result is exact, and rescaling is rare.
#include <math.h>

#include "rglru_device.h"
#include "rglru_internal.h"
#include "rglru_lds_copy.h"

namespace rglru {
namespace {

constexpr int kDh = 256;       // head dimension
constexpr int kQB = 128;       // queries per workgroup (4 waves of 32)
constexpr int kKB = 32;        // keys per tile
constexpr int kAttnThreads = 256;
constexpr float kRescale = 8.0f;  // exp2 units: rescale when a tile maximum exceeds the reference by 2^8

// ---------------------------------------------------------------------------------------
// Ring KV cache for decoding.  Per sequence, Wc / 32 tiles of 32 slots x 256 dims (16 KB of K and
// 16 KB of V each); slot t % W holds position t.  Within a tile both are stored in the operand
// order of v_mfma_f32_16x16x32_bf16 (lane l supplies row l % 16 and K-slice l / 16 of 8), so
// that one fragment of a wave is 1 KB of contiguous memory:
//   K, the A operand of S^T = K Q^T (rows: slots, K: dims), fragment (half, kk) for slots
//   16 half .. + 15 and dims 32 kk .. + 31;
//   V, the A operand of O^T = V^T P^T (rows: dims, K: slots), fragment jd for dims 16 jd .. + 15;
//   lane group g = l / 16 holds slots 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3, the slots whose
//   scores the same lane holds in the two S^T results (rows 4 g + i of each).
// ---------------------------------------------------------------------------------------
constexpr int kTileElems = 32 * kDh;   // elements of one cache tile (K or V)

__device__ __forceinline__ int kc_index(int r, int d) {  // slot r of a tile, dim d
    return ((((r >> 4) * 8 + (d >> 5)) * 4 + ((d & 31) >> 3)) * 16 + (r & 15)) * 8 + (d & 7);
}
__device__ __forceinline__ int vc_index(int r, int d) {
    const int rr = r & 15;
    return (((d >> 4) * 4 + (rr >> 2)) * 16 + (d & 15)) * 8 + (rr & 3) + 4 * (r >> 4);
}

// ---------------------------------------------------------------------------------------
// prep: one workgroup per token row t in [0, 4 ceil(T / 4)) of one sequence
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) attn_prep_kernel(AttnArgs a) {
    const int rows = 4 * a.T4;
    const int b = blockIdx.x / rows, t = blockIdx.x % rows;
    const int tid = threadIdx.x;
    const bool valid = t < a.T;
    const size_t m = (size_t)b * a.T + (valid ? t : 0);
    // v, regrouped: v4[b][t / 4][d][t % 4]; rows past T are zero (their weight is 0, but a
    // non-finite value times 0 would not be)
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    uint16_t* v4 = static_cast<uint16_t*>(a.v4);
    v4[(((size_t)b * a.T4 + t / 4) * kDh + tid) * 4 + (t & 3)] = valid ? v[m * kDh + tid] : 0;
    if (!valid) return;
    // the last W positions also go to the ring cache, if one is given
    const bool to_cache = a.kc != nullptr && t >= a.T - a.W;
    const int slot = t % a.W;
    const size_t ctile = ((size_t)b * (a.Wc / 32) + slot / 32) * kTileElems;
    if (to_cache)
        static_cast<uint16_t*>(a.vc)[ctile + vc_index(slot & 31, tid)] = v[m * kDh + tid];
    // RoPE: pair i of a head, (x_i, x_{i+128}), turned by t * base^(-2 i / 256)
    const int HD = a.Hq * kDh;
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + m * HD;
    const uint16_t* k = static_cast<const uint16_t*>(a.k) + m * kDh;
    uint16_t* qr = static_cast<uint16_t*>(a.qr) + m * HD;
    uint16_t* kr = static_cast<uint16_t*>(a.kr) + m * kDh;
    // the angle depends on (t, i) only: thread tid turns pair i = tid % 128 of heads
    // tid / 128, tid / 128 + 2, ... (the key head counted as head Hq)
    const int i = tid % (kDh / 2);
    const double ang = (double)t * exp2(-2.0 * (double)i / (double)kDh * log2((double)a.rope_base));
    double sn_d, cs_d;
    sincos(ang, &sn_d, &cs_d);
    const float sn = (float)sn_d, cs = (float)cs_d;
    for (int h = tid / (kDh / 2); h <= a.Hq; h += 2) {
        const uint16_t* src = h < a.Hq ? q + h * kDh : k;
        uint16_t* dst = h < a.Hq ? qr + h * kDh : kr;
        const float x0 = bf2f(src[i]), x1 = bf2f(src[i + kDh / 2]);
        const uint16_t r0 = f2bf(x0 * cs - x1 * sn), r1 = f2bf(x1 * cs + x0 * sn);
        dst[i] = r0;
        dst[i + kDh / 2] = r1;
        if (h == a.Hq && to_cache) {
            uint16_t* kc = static_cast<uint16_t*>(a.kc) + ctile;
            kc[kc_index(slot & 31, i)] = r0;
            kc[kc_index(slot & 31, i + kDh / 2)] = r1;
        }
    }
}

// ---------------------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------------------
// x *= f for a value held in an accumulation register.  Written out so that the output
// accumulators stay in AGPRs across the key loop: left to itself, the compiler moved all of them
// to VGPRs and back on every tile for the sake of this rarely taken multiply.
__device__ __forceinline__ void scale_acc(float& x, float f) {
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\t"
                 "v_mul_f32 %1, %1, %2\n\t"
                 "v_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(t)
                 : "v"(f));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One K/V tile of 32 keys, copied straight into an LDS stage: each wave issues 8 copies of
// 1 KB, 4 of K and 4 of V, lane l of copy i filling stage chunk p = 64 (4 wave + i) + l.
//   K stage: [key][32 chunks of 8 dims]; chunk c of key r sits at position c ^ (r % 16), so the
//   16 lanes of a fragment read (16 keys, one chunk index) hit 16 distinct bank groups.
//   V stage: 8 groups of 4 keys x 256 dims x 4 keys, a contiguous 16 KB slice of v4.
// Keys past T repeat the last key (finite; their weight is 0).  rk / rv address one sequence's
// k and v4.
__device__ __forceinline__ void copy_tile(const u32x4& rk, const u32x4& rv, uint16_t* kl,
                                          uint16_t* vl, int T, int T4, int kt, int wv, int lane) {
    int ok[4], ov[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = (4 * wv + i) * 64 + lane;
        const int key = p >> 5, pos = p & 31;
        const int c = pos ^ (key & 15);
        ok[i] = (min(kt * kKB + key, T - 1) * kDh + c * 8) * 2;
        const int g = min(kt * (kKB / 4) + (p >> 7), T4 - 1);
        ov[i] = (g * (kDh * 4) + (p & 127) * 8) * 2;
    }
    copy4(rk, lds_address(kl + 4 * wv * 512), ok);
    copy4(rv, lds_address(vl + 4 * wv * 512), ov);
}

// Four consecutive bf16 keys of one dimension (8 bytes) from a V stage.
__device__ __forceinline__ uint2 v_quad(const uint16_t* vl, int g, int d) {
    return *reinterpret_cast<const uint2*>(vl + (g * kDh + d) * 4);
}

__global__ void __launch_bounds__(kAttnThreads, 1) attn_fwd_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t k0[kKB * kDh], k1[kKB * kDh];
    __shared__ __attribute__((aligned(16))) uint16_t v0[kKB * kDh], v1[kKB * kDh];

    const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nqb = (a.T + kQB - 1) / kQB;
    const int qb = blockIdx.x % nqb;
    const int bh = blockIdx.x / nqb;
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int q0 = qb * kQB;
    const int t0w = q0 + 32 * wv;                  // this wave's first query
    const int tq = t0w + (lane & 31);              // this lane's query
    const int W = a.W, T = a.T;

    // Q fragments (B operand of S^T = K Q^T): query tq, dims 16 kk + 8 hl .. + 7
    bf16x8 qf[16];
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.qr) +
                               ((size_t)b * T + min(tq, T - 1)) * ((size_t)a.Hq * kDh) + h * kDh;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * hl);
    }

    f32x16 oacc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[j][e] = 0.0f;
    float mref = -1e30f;                            // reference maximum (exp2 units)
    float lsum = 0.0f;                              // this lane's share of the normaliser
    const float sc = kLog2e * 0.0625f;              // log2(e) / sqrt(256)

    const int klo = max(0, q0 - W + 1);
    const int khi = min(T - 1, q0 + kQB - 1);
    const int ktlo = klo / kKB, kthi = khi / kKB;
    // this wave's live tiles, kta .. ktb: those holding a key of some query's window, keys
    // t0w - W + 1 .. t0w + 31 (none for a wave past the end of the sequence)
    const int ktb = t0w < T ? min(kthi, t0w / kKB) : ktlo - 1;
    const int kta = max(ktlo, max(0, t0w - W + 1) / kKB);

    const uint16_t* kseq = static_cast<const uint16_t*>(a.kr) + (size_t)b * T * kDh;
    const uint16_t* vseq = static_cast<const uint16_t*>(a.v4) + (size_t)b * a.T4 * (kDh * 4);
    const u32x4 rk = rsrc_words(kseq, (uint32_t)T * kDh * 2);
    const u32x4 rv = rsrc_words(vseq, (uint32_t)a.T4 * kDh * 4 * 2);
    guard_vmem_sgprs(rk, rv);
    // Q fragments are loaded (and waited for) before the first copy: from here on the copies
    // are this wave's only vector-memory instructions until the stores at the end.
    __builtin_amdgcn_s_waitcnt(0x0f70);
    copy_tile(rk, rv, k0, v0, T, a.T4, ktlo, wv, lane);

    // One step per key tile, the same count on every wave: this wave's copies of tile kt (the
    // only ones in flight) have landed; after the barrier every wave's have, and every wave is
    // done with tile kt - 1, whose stage takes kt + 1.
    auto advance = [&](int kt) {
        wait_vmcnt<0>();
        lds_sync();
        if (kt + 1 <= kthi) {
            const bool odd = ((kt - ktlo) & 1) != 0;
            copy_tile(rk, rv, odd ? k0 : k1, odd ? v0 : v1, T, a.T4, kt + 1, wv, lane);
        }
    };
    // The three loops keep the tile computation free of a skip branch: with one, the
    // compiler carried the output accumulators through VGPRs and copied all of them on every
    // tile.
    int kt = ktlo;
    for (; kt < kta; ++kt) advance(kt);
    for (; kt <= ktb; ++kt) {
        advance(kt);
        const bool odd = ((kt - ktlo) & 1) != 0;
        const uint16_t* kc = odd ? k1 : k0;
        const uint16_t* vc = odd ? v1 : v0;
        const int key0 = kt * kKB;
        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.0f;
        const int kr_ = lane & 31;
        // fragment reads in groups of four, so that at most eight are in flight (left free,
        // the compiler hoisted all of them and ran out of registers)
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int pos = (2 * kk + hl) ^ (kr_ & 15);
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kc + kr_ * kDh + pos * 8);
            s = mfma32(kf, qf[kk], s);
            if ((kk & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = s[e] * sc;
        // mask only on tiles that cross a window edge or the sequence end
        if (key0 + kKB - 1 > t0w || key0 <= t0w + 31 - W || key0 + kKB > T) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = key0 + mfma_d_row(lane, e);
                x[e] = (key > tq || key <= tq - W || key >= T) ? -INFINITY : x[e];
            }
        }
        float tmax = x[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, x[e]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool need = tmax > mref + kRescale;
        if (__any(need)) {
            const float al = need ? __builtin_amdgcn_exp2f(mref - tmax) : 1.0f;
            if (need) mref = tmax;
            lsum *= al;
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float y = oacc[j][e];
                    scale_acc(y, al);
                    oacc[j][e] = y;
                }
        }
        float p[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            p[e] = __builtin_amdgcn_exp2f(x[e] - mref);
            lsum += p[e];
        }
        bf16x8 pf[2];
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
            for (int i = 0; i < 8; ++i) pf[kq][i] = (__bf16)p[8 * kq + i];
        // O^T[j] += V^T P^T: dims 32 j + l % 32; keys 16 kq + 4 hl + {0..3} and {8..11}
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int d = 32 * j + (lane & 31);
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                const uint2 lo = v_quad(vc, 4 * kq + hl, d);
                const uint2 hi = v_quad(vc, 4 * kq + hl + 2, d);
                const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                oacc[j] = mfma32(vf, pf[kq], oacc[j]);
            }
            if ((j & 1) == 1) __builtin_amdgcn_sched_barrier(0);
        }
    }
    for (; kt <= kthi; ++kt) advance(kt);

    // normalise and store: O^T tile j, register 4 g + i -> dim 32 j + 8 g + 4 hl + i
    const float lt = lsum + __shfl_xor(lsum, 32);
    const float inv = 1.0f / lt;
    if (tq < T) {
        uint16_t* orow = static_cast<uint16_t*>(a.o) + ((size_t)b * T + tq) * ((size_t)a.Hq * kDh) +
                         h * kDh;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * j + 8 * g + 4 * hl;
                *reinterpret_cast<uint2*>(orow + d) =
                    make_uint2(pack2bf(oacc[j][4 * g] * inv, oacc[j][4 * g + 1] * inv),
                               pack2bf(oacc[j][4 * g + 2] * inv, oacc[j][4 * g + 3] * inv));
            }
    }
}

// ---------------------------------------------------------------------------------------
// decode: one new token per sequence
// ---------------------------------------------------------------------------------------
// RoPE of the new token's q and k at its position; k and v go to cache slot pos % W.
__global__ void __launch_bounds__(256) attn_dec_prep_kernel(AttnDecodeArgs a) {
    const int n = blockIdx.x, tid = threadIdx.x;
    const int t = a.pos[n];
    if (t < 0) return;
    const int slot = t % a.W;
    const size_t ctile = ((size_t)n * (a.Wc / 32) + slot / 32) * kTileElems;
    static_cast<uint16_t*>(a.vc)[ctile + vc_index(slot & 31, tid)] =
        static_cast<const uint16_t*>(a.v)[(size_t)n * kDh + tid];
    const int i = tid % (kDh / 2);
    const double ang = (double)t * exp2(-2.0 * (double)i / (double)kDh * log2((double)a.rope_base));
    double sn_d, cs_d;
    sincos(ang, &sn_d, &cs_d);
    const float sn = (float)sn_d, cs = (float)cs_d;
    for (int h = tid / (kDh / 2); h <= a.Hq; h += 2) {
        const uint16_t* src = h < a.Hq
            ? static_cast<const uint16_t*>(a.q) + ((size_t)n * a.Hq + h) * kDh
            : static_cast<const uint16_t*>(a.k) + (size_t)n * kDh;
        const float x0 = bf2f(src[i]), x1 = bf2f(src[i + kDh / 2]);
        const uint16_t r0 = f2bf(x0 * cs - x1 * sn), r1 = f2bf(x1 * cs + x0 * sn);
        if (h < a.Hq) {
            uint16_t* dst = static_cast<uint16_t*>(a.qr) + ((size_t)n * a.Hq + h) * kDh;
            dst[i] = r0;
            dst[i + kDh / 2] = r1;
        } else {
            uint16_t* kc = static_cast<uint16_t*>(a.kc) + ctile;
            kc[kc_index(slot & 31, i)] = r0;
            kc[kc_index(slot & 31, i + kDh / 2)] = r1;
        }
    }
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One workgroup per (sequence, 128 TPW cache slots): each wave takes TPW (1, 2 or 4) 32-slot tiles
// (tile 4 TPW sp + 4 i + wave, i < TPW), heads as the 16 columns of S^T = K Q^T and O^T = V^T P^T, and a softmax
// per head over its tiles; the four waves are merged through LDS into one partial result
// (reference maximum M, normaliser L, unnormalised output O) per head.  Only slots below
// min(pos + 1, W) hold positions of the window; the others are masked, and their V entries
// zeroed (a slot never written may hold any bits).
constexpr int kDecPad = 260;   // LDS row pitch (floats) of the per-wave outputs
template <int TPW>
__global__ void __launch_bounds__(256, 2) attn_dec_kernel(AttnDecodeArgs a) {
    __shared__ __attribute__((aligned(16))) float ow[4][16][kDecPad];
    __shared__ float wm[4][16], wl[4][16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = blockIdx.x / a.nsplit, sp = blockIdx.x % a.nsplit;
    const int col = lane & 15, g = lane >> 4;
    const int t = a.pos[n];
    const int nvalid = t < 0 ? 0 : min(t + 1, a.W);

    bf16x8 qf[8];
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.qr) +
                               ((size_t)n * a.Hq + min(col, a.Hq - 1)) * kDh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * g);
            if (col >= a.Hq) qf[kk] = bf16x8{};
        }
    }
    f32x4 oacc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float sc = kLog2e * 0.0625f;
    const uint16_t* kseq = static_cast<const uint16_t*>(a.kc) + (size_t)n * (a.Wc / 32) * kTileElems;
    const uint16_t* vseq = static_cast<const uint16_t*>(a.vc) + (size_t)n * (a.Wc / 32) * kTileElems;

    int ntile = 0;   // this wave's tiles holding a slot of the window (a prefix of its TPW)
#pragma unroll
    for (int i = 0; i < TPW; ++i) ntile += ((sp * 4 * TPW + 4 * i + wv) * 32 < nvalid) ? 1 : 0;

    // Pass 1: scores of the wave's tiles, kept in registers, and their exact maximum per head
    // (no running rescale; no branch surrounds the accumulating MFMAs).
    // xs[i][m]: tile i, slot 4 g + m (m < 4) or 16 + 4 g + m - 4, the order of the P^T operand.
    // A tile's 16 fragments (16 KB per wave) are loaded together, the next tile's before this
    // tile's MFMAs (two register buffers), and the first value tile's during the last key tile
    // (one buffer for the values: the output accumulators take the registers); the scheduling
    // barriers keep the compiler from sinking each load next to its use, which left
    // only two to four fragments of a wave in flight.  The loads are unconditional (a branch
    // around them makes the compiler's wait counts fall back to waiting for all): a tile past
    // the wave's live ones re-reads its first tile, clamped to the last tile holding a slot of
    // the window (cache hits; its scores and values are discarded below).
    const int last_tile = (nvalid > 0 ? nvalid - 1 : 0) / 32;
    auto load_tile = [&](bf16x8* f16, const uint16_t* base, int i) {
        const int tile = min(sp * 4 * TPW + 4 * (i < ntile ? i : 0) + wv, last_tile);
        const uint16_t* tp = base + (size_t)tile * kTileElems;
#pragma unroll
        for (int f = 0; f < 16; ++f)
            f16[f] = *reinterpret_cast<const bf16x8*>(tp + (f * 64 + lane) * 8);
    };
    float xs[TPW][8];
    float mx = -INFINITY;
    bf16x8 kf[2][16], vf[16];
    load_tile(kf[0], kseq, 0);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tile = sp * 4 * TPW + 4 * i + wv, s0 = tile * 32;
        if (i + 1 < TPW) load_tile(kf[(i + 1) & 1], kseq, i + 1);
        else load_tile(vf, vseq, 0);
        __builtin_amdgcn_sched_barrier(0);
        {
            const bf16x8* kc = kf[i & 1];
            f32x4 sa = {0.0f, 0.0f, 0.0f, 0.0f}, sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                sa = mfma16(kc[kk], qf[kk], sa);
                sb = mfma16(kc[8 + kk], qf[kk], sb);
            }
            const bool live = i < ntile;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                xs[i][m] = live ? sa[m] * sc : -INFINITY;
                xs[i][4 + m] = live ? sb[m] * sc : -INFINITY;
            }
            if (live && s0 + 32 > nvalid) {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    if (s0 + (m < 4 ? 4 * g + m : 16 + 4 * g + m - 4) >= nvalid) xs[i][m] = -INFINITY;
            }
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) mx = fmaxf(mx, xs[i][m]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mref = fmaxf(mx, -1e30f);   // a wave without tiles keeps a finite reference
    float lsum = 0.0f;

    // Pass 2: O^T += V^T P^T over the same tiles; a tile past the window contributes zeros
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tile = sp * 4 * TPW + 4 * i + wv, s0 = tile * 32;
        if (i > 0) load_tile(vf, vseq, i);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8* vc = vf;
        if (i < ntile) {
            if (s0 + 32 > nvalid) {
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const bool dead = s0 + (m < 4 ? 4 * g + m : 16 + 4 * g + m - 4) >= nvalid;
#pragma unroll
                    for (int f = 0; f < 16; ++f) vc[f][m] = dead ? (__bf16)0.0f : vc[f][m];
                }
            }
        } else {
#pragma unroll
            for (int f = 0; f < 16; ++f) vc[f] = bf16x8{};
        }
        bf16x8 pf;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float p = __builtin_amdgcn_exp2f(xs[i][m] - mref);
            lsum += p;
            pf[m] = (__bf16)p;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[j] = mfma16(vc[j], pf, oacc[j]);
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    // O^T fragment j: column col, dims 16 j + 4 g + e
#pragma unroll
    for (int j = 0; j < 16; ++j)
        *reinterpret_cast<f32x4*>(&ow[wv][col][16 * j + 4 * g]) = oacc[j];
    if (g == 0) {
        wm[wv][col] = mref;
        wl[wv][col] = lsum;
    }
    __syncthreads();
    float* prow = a.part + ((size_t)n * a.nsplit + sp) * a.Hq * (2 + kDh);
    const int d = tid;
    for (int h = 0; h < a.Hq; ++h) {
        const float M = fmaxf(fmaxf(wm[0][h], wm[1][h]), fmaxf(wm[2][h], wm[3][h]));
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = __builtin_amdgcn_exp2f(wm[w][h] - M);
            L += f * wl[w][h];
            O += f * ow[w][h][d];
        }
        prow[(size_t)h * (2 + kDh) + 2 + d] = O;
        if (d == 0) {
            prow[(size_t)h * (2 + kDh)] = M;
            prow[(size_t)h * (2 + kDh) + 1] = L;
        }
    }
}

// o[n][h] = sum over splits of 2^(M_s - M) O_s / sum of 2^(M_s - M) L_s, in split order.
__global__ void __launch_bounds__(256) attn_dec_combine_kernel(AttnDecodeArgs a) {
    const int n = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq, d = threadIdx.x;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + ((size_t)n * a.Hq + h) * kDh;
    if (a.pos[n] < 0) {
        orow[d] = 0;
        return;
    }
    const float* p0 = a.part + ((size_t)n * a.nsplit * a.Hq + h) * (2 + kDh);
    const size_t stride = (size_t)a.Hq * (2 + kDh);
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, p0[s * stride]);
    float L = 0.0f, O = 0.0f;
    for (int s = 0; s < a.nsplit; ++s) {
        const float f = __builtin_amdgcn_exp2f(p0[s * stride] - M);
        L += f * p0[s * stride + 1];
        O += f * p0[s * stride + 2 + d];
    }
    orow[d] = f2bf(O / L);
}

}  // namespace

hipError_t launch_attention_decode(const AttnDecodeArgs& a, hipStream_t s) {
    if (a.N == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_dec_prep_kernel, dim3((unsigned)a.N), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(a.N * a.nsplit));
    switch (a.tpw) {
        case 1: hipLaunchKernelGGL(attn_dec_kernel<1>, grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL(attn_dec_kernel<2>, grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL(attn_dec_kernel<4>, grid, dim3(256), 0, s, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_dec_combine_kernel, dim3((unsigned)(a.N * a.Hq)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_prep_kernel, dim3((unsigned)(a.B * 4 * a.T4)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long blocks = (long long)a.B * a.Hq * ((a.T + kQB - 1) / kQB);
    hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)blocks), dim3(kAttnThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace rglru
