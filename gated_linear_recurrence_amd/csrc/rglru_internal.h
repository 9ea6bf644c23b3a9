// Host-side declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rglru {

constexpr int kSeg = 64;              // tokens per prefill time segment (one workgroup)
constexpr size_t kWsHeader = 4096;    // workspace header bytes (counters and error flags)
// header words: [0] error flags of the latest call, [kTicketWord + h] ticket counter of head h;
// every prefill call clears the header and the carry words it uses before its scan kernel runs
constexpr int kErrWord = 0;
constexpr int kTicketWord = 16;
constexpr size_t kZeroBlock = 2048;  // the ticket counters end before header byte 2048
constexpr int kMaxHeads = (int)(kZeroBlock / 4) - kTicketWord;

struct PrefillArgs {
    const void* x;
    const void* y;
    void* out;
    const void* conv_w;
    const void* conv_b;
    const void* wa;
    const void* ba;
    const void* wx;
    const void* bx;
    const float* lambda;
    const float* h0;
    float* h_last;
    const void* conv0;
    void* conv_last;
    unsigned long long* words;  // carry words [S][B][D]
    unsigned* header;           // see kErrWord, kTicketWord
    int B, T, D, H, S;
    int n_units;                // S * B * H units (generic kernel: one workgroup each)
    int wph;                    // persistent kernel: workgroups per head
};

struct DecodeArgs {
    const void* x;
    const void* y;
    void* out;
    long long ld_x, ld_y, ld_out;
    const void* conv_w;
    const void* conv_b;
    const void* wa;
    const void* ba;
    const void* wx;
    const void* bx;
    const float* lambda;
    float* h;
    void* conv_state;
    void* u_ws;  // split decode: u [N][D] in the storage dtype, or NULL for the fused kernel
    int N, D, H;
};

struct ConvArgs {
    const void* x;       // [N][T][D]
    const void* conv_w;
    const void* conv_b;
    void* conv_state;    // [N][3][D]
    void* conv_out;      // [N][T][D] or null
    int N, T, D;
};

// One Linear layer, or up to three side by side over the same input (the block's branch
// projections; the attention block's q, k and v), as a bf16 GEMM: output segment o has width
// Nw[o] and C_o[m][n] = b_o[n] + sum_k A[m][k] W_o[n][k], each C_o [M][Nw[o]].
struct ProjGemmArgs {
    const void* A;               // [M][K]
    const void* W[3];            // [Nw[o]][K]
    const void* b[3];            // [Nw[o]] or null
    void* C[3];                  // [M][Nw[o]]
    int Nw[3];                   // multiples of 256 (unused segments 0)
    int nseg;                    // 1 .. 3
    int M, K;                    // K % 128 == 0, 256 * Nw < 2^31
    int ntm, ntn;                // set by the launcher
    // split K (small M): with part given, the launcher may split K in up to part_bytes of fp32
    // partial sums [ksplit][M][sum Nw], added in split order by a second kernel
    float* part;
    size_t part_bytes;
    int ksplit;                  // set by the launcher
    int c_f32;                   // split-K only: C[0] is fp32 (no rounding); the call fails
                                 // unless the launcher splits K
    // gated: proj_gemm_gated_ok(M, K); R: the row kernel, or any shape with rows_epilogue; the
    // call fails otherwise.
    int gated;                   // two segments of equal width: C[0] = gelu_tanh(gate) * up,
                                 // from the bf16-rounded segment outputs (C[1] unused)
    const void* R;               // one segment: C = R + the rounded output, rounded again
    // rows_epilogue (one segment of at most 8192 columns, M > 4, part given): the tile
    // kernels write fp32 partials even without a K split, and one workgroup per row adds them
    // with the bias and R, and, with norm_out, also writes RMSNorm(C) * norm_g (the
    // add-and-norm step of the residual layer)
    int rows_epilogue;
    const void* norm_g;
    void* norm_out;
    float norm_eps;
    // in_norm_g (the row kernel only; the call fails otherwise): A holds the rows before an
    // RMSNorm of scale in_norm_g [K] and the kernel multiplies by RMSNorm(A row) * in_norm_g,
    // each element rounded to bf16 as the norm kernel would write it
    const void* in_norm_g;
    float in_norm_eps;
    // Tile kernel only: `batch` (>= 1; 0 means 1) independent GEMMs of this shape in one launch,
    // item i at A + i bsA, W[o] + i bsW, C[o] + i bsC, b[o] + i bsb (elements), with its own
    // split-K partials [ksplit][M][sum Nw] at part + i ksplit M sum Nw.
    int batch;
    long long bsA, bsW, bsC, bsb;
};
// true when launch_proj_gemm takes the row kernel (which supports gated and R)
bool proj_gemm_rows(int M, int K);
// true when a GEMM of M rows may be gated: the row kernel, or the mid-size tiles (5..1024 rows)
bool proj_gemm_gated_ok(int M, int K);
// fp32 partial-sum bytes the launcher would use for this shape with unlimited part_bytes
size_t proj_gemm_part_bytes(int M, int Ntot, int K);
// true when a GEMM of M rows can take rows_epilogue (the tile kernels: M > 4)
bool proj_gemm_rows_epilogue_ok(int M);
// the partial-sum bytes of that form (at least one split's worth)
size_t proj_gemm_part_bytes_rows_epilogue(int M, int Ntot, int K);
// the same for `batch` GEMMs of this shape in one launch (tile kernel)
size_t proj_gemm_part_bytes_batched(int batch, int M, int Ntot, int K);

// Local sliding-window multi-query attention (head dim 256).
struct AttnArgs {
    const void* q;       // [B][T][Hq * 256] before RoPE
    const void* k;       // [B][T][256]
    const void* v;       // [B][T][256]
    void* qr;            // workspace: q after RoPE
    void* kr;            // workspace: k after RoPE
    void* v4;            // workspace: v regrouped [B][T4][256][4]
    void* o;             // [B][T][Hq * 256]
    void* kc;            // optional ring caches [B][Wc / 32][16 KB] (NULL: not filled)
    void* vc;
    int B, T, Hq, W, T4; // T4 = ceil(T / 4)
    int Wc;              // cache slots per sequence, W rounded up to 32
    float rope_base;
};

// One decode step of local attention for N sequences.
struct AttnDecodeArgs {
    const int* pos;      // [N] position of the new token (device)
    const void* q;       // [N][Hq * 256] before RoPE
    const void* k;       // [N][256]
    const void* v;       // [N][256]
    void* kc;            // ring caches [N][Wc / 32][16 KB]
    void* vc;
    void* qr;            // workspace: q after RoPE [N][Hq][256]
    float* part;         // workspace: partial results [N][nsplit][Hq][2 + 256]
    void* o;             // [N][Hq * 256]
    int N, Hq, W, Wc, nsplit;
    int tpw;             // 32-slot tiles per wave (1, 2 or 4): 128 tpw slots per split
    float rope_base;
};

int device_cu_count();  // compute units of the current device (cached)
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int bs, hipStream_t s);
hipError_t launch_prefill_empty(const PrefillArgs& a, int dtype, hipStream_t s);
hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int bs, hipStream_t s);
hipError_t launch_conv_update(const ConvArgs& a, int dtype, hipStream_t s);
hipError_t launch_proj_gemm(const ProjGemmArgs& a, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_decode(const AttnDecodeArgs& a, hipStream_t s);

// Residual-layer elementwise steps (bf16): h = x (+ y) and n = RMSNorm(h) * g over rows of D.
struct NormArgs {
    const void* x;       // [M][D]
    const void* y;       // [M][D] or NULL
    const void* g;       // [D] (needed when n is given)
    void* h;             // [M][D] or NULL: x + y rounded to bf16
    void* n;             // [M][D] or NULL
    int M, D;            // D % 8 == 0, D <= 8192
    float eps;
};
hipError_t launch_add_rmsnorm(const NormArgs& a, hipStream_t s);

// Backward pass of the path (bf16 storage, block size 256, T % 32 == 0, B * T % 256 == 0).
struct BwdArgs {
    const void *x, *y, *dout;            // [B][T][D] bf16
    const float* h0;                     // [B][D] or NULL
    const void* conv0;                   // [B][3][D] bf16 or NULL
    const float* dh_last;                // [B][D] or NULL
    const void *conv_w, *conv_b, *wa, *ba, *wx, *bx;
    const float* lambda;
    void *dx, *dy;                       // [B][T][D] bf16
    float *dconv_w, *dconv_b, *dwa, *dba, *dwx, *dbx, *dlambda, *dh0, *dconv0;
    void* ws;                            // workspace (rglru_prefill_backward_workspace_bytes)
    int B, T, D, H;
};
size_t backward_workspace_bytes(int B, int T, int D, int H);
hipError_t launch_prefill_backward(const BwdArgs& a, hipStream_t s);
hipError_t launch_geglu(void* gate, const void* up, size_t n, hipStream_t s);  // n % 8 == 0
// Decode attention: 32-slot tiles per wave (four waves per workgroup, so 128 tpw cache slots per
// workgroup).  Four for batches of 64 or more; fewer for small batches, whose windows would
// otherwise be read by only a few compute units.
inline int attn_dec_tiles_per_wave(long long N) { return N >= 64 ? 4 : (N >= 16 ? 2 : 1); }
inline long long attn_dec_nsplit(long long N, long long window) {
    const long long slots = 128LL * attn_dec_tiles_per_wave(N);
    return (window + slots - 1) / slots;
}

}  // namespace rglru
