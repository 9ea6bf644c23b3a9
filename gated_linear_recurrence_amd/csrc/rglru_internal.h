// Host-side declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rglru {

constexpr int kSeg = 64;              // tokens per prefill time segment (one workgroup)
constexpr size_t kWsHeader = 4096;    // workspace header bytes (counters and error flags)
// header words: [0] error flags, [1] finished workgroups, [kTicketWord + h] ticket counter of head h
constexpr int kErrWord = 0;
constexpr int kDoneWord = 1;
constexpr int kTicketWord = 16;
constexpr size_t kZeroBlock = 2048;  // header bytes [2048, 4096) stay zero: a zero source for copies
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
    unsigned* header;           // see kErrWord, kDoneWord, kTicketWord
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

// One Linear layer (or the two branch projections side by side) as a bf16 GEMM:
// C_o[m][n] = b_o[n] + sum_k A[m][k] W_o[n][k] for output o < n_out, each [M][N0].
struct ProjGemmArgs {
    const void* A;               // [M][K]
    const void* W0;              // [N0][K]
    const void* W1;              // [N0][K] (n_out == 2) or null
    const void* b0;              // [N0] or null
    const void* b1;
    void* C0;                    // [M][N0]
    void* C1;
    int M, K, N0, n_out;         // N0 % 256 == 0, K % 128 == 0, 256 * N0 < 2^31
    int ntm, ntn;                // set by the launcher
};

int device_cu_count();  // compute units of the current device (cached)
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int bs, hipStream_t s);
hipError_t launch_prefill_empty(const PrefillArgs& a, int dtype, hipStream_t s);
hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int bs, hipStream_t s);
hipError_t launch_conv_update(const ConvArgs& a, int dtype, hipStream_t s);
hipError_t launch_proj_gemm(const ProjGemmArgs& a, hipStream_t s);

}  // namespace rglru
