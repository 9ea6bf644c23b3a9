// C ABI of librglru.so: argument validation, workspace sizing and kernel launches.
// Every check runs on the host before any HIP call; see include/rglru.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/rglru.h"
#include "rglru_internal.h"

using namespace rglru;

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return RGLRU_ERR_HIP;
}

size_t elem_size(int dtype) { return dtype == RGLRU_BF16 ? 2 : 4; }

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

constexpr int kAttnDh = 256;  // the attention's head width

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

// [p, p + n) and [q, q + m) overlap (null or empty ranges never overlap)
bool overlap(const void* p, size_t n, const void* q, size_t m) {
    if (!p || !q || n == 0 || m == 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + m && b < a + n;
}

// Shared checks of the parameter struct.  Returns RGLRU_OK or an error status.
int check_params(const rglru_params* p, bool need_gates) {
    if (!p) return RGLRU_ERR_NULL;
    if (p->dtype != RGLRU_F32 && p->dtype != RGLRU_BF16) return RGLRU_ERR_UNSUPPORTED;
    if (p->D < 1 || p->n_heads < 1 || p->D % p->n_heads != 0) return RGLRU_ERR_SHAPE;
    if (!p->conv_w) return RGLRU_ERR_NULL;
    if (!aligned16(p->conv_w) || !aligned16(p->conv_b)) return RGLRU_ERR_UNSUPPORTED;
    if (p->D % 8 != 0) return RGLRU_ERR_UNSUPPORTED;
    if (need_gates) {
        const int bs = p->D / p->n_heads;
        if (bs != 128 && bs != 256) return RGLRU_ERR_UNSUPPORTED;
        if (p->n_heads > kMaxHeads) return RGLRU_ERR_UNSUPPORTED;
        if (!p->gate_a_w || !p->gate_x_w || !p->lambda) return RGLRU_ERR_NULL;
        if (!aligned16(p->gate_a_w) || !aligned16(p->gate_x_w) || !aligned16(p->gate_a_b) ||
            !aligned16(p->gate_x_b) || !aligned16(p->lambda))
            return RGLRU_ERR_UNSUPPORTED;
    }
    return RGLRU_OK;
}

size_t n_segments(int32_t T) { return T <= 0 ? 1 : ((size_t)T + kSeg - 1) / kSeg; }

}  // namespace

extern "C" {

int rglru_abi_version(void) { return RGLRU_ABI_VERSION; }

int rglru_last_hip_error(void) { return g_last_hip_error; }

const char* rglru_status_string(int status) {
    switch (status) {
        case RGLRU_OK: return "ok";
        case RGLRU_ERR_NULL: return "a required pointer is NULL";
        case RGLRU_ERR_SHAPE: return "invalid shape";
        case RGLRU_ERR_UNSUPPORTED: return "unsupported block size, dtype or alignment";
        case RGLRU_ERR_WORKSPACE: return "workspace missing or too small";
        case RGLRU_ERR_ALIAS: return "an output overlaps an input it may not alias";
        case RGLRU_ERR_HIP: return "HIP call failed";
        default: return "unknown status";
    }
}

size_t rglru_prefill_workspace_bytes(int32_t B, int32_t T, int32_t D, int32_t n_heads,
                                     int32_t dtype) {
    if (B < 1 || T < 0 || D < 1 || n_heads < 1 || D % n_heads != 0) return 0;
    if (dtype != RGLRU_F32 && dtype != RGLRU_BF16) return 0;
    // carry words of every segment but the last (which publishes none)
    return kWsHeader + (n_segments(T) - 1) * (size_t)B * (size_t)D * sizeof(unsigned long long);
}

int rglru_prefill_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
    if (!workspace) return RGLRU_ERR_NULL;
    if (!aligned16(workspace)) return RGLRU_ERR_UNSUPPORTED;
    if (ws_bytes < kWsHeader) return RGLRU_ERR_WORKSPACE;
    hipError_t e = launch_workspace_init(workspace, ws_bytes, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// Every check rglru_prefill makes before it launches anything.
// static_ws: the look-back state lives in the library's static scratch (rglru_prefill_noalloc),
// so the workspace arguments are not checked here.
int check_prefill(const rglru_params* p, int32_t B, int32_t T, const void* x, const void* y,
                  void* out, const float* h0, float* h_last, const void* conv0, void* conv_last,
                  void* workspace, size_t ws_bytes, bool static_ws = false) {
    int st = check_params(p, true);
    if (st != RGLRU_OK) return st;
    if (B < 1 || T < 0) return RGLRU_ERR_SHAPE;
    if (T > 0 && (!x || !y || !out)) return RGLRU_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(out) || !aligned16(h0) ||
        !aligned16(h_last) || !aligned16(conv0) || !aligned16(conv_last) || !aligned16(workspace))
        return RGLRU_ERR_UNSUPPORTED;
    const size_t es = elem_size(p->dtype);
    // the bf16 kernel addresses one sequence's rows, and the carried conv window of all
    // sequences, with 32-bit byte offsets
    if (p->dtype == RGLRU_BF16 && ((size_t)T * (size_t)p->D * es >= ((size_t)1 << 31) ||
                                   (size_t)B * 3 * (size_t)p->D * es >= ((size_t)1 << 31)))
        return RGLRU_ERR_UNSUPPORTED;
    const size_t n_act = (size_t)B * (size_t)T * (size_t)p->D * es;
    const size_t n_h = (size_t)B * (size_t)p->D * sizeof(float);
    const size_t n_c = (size_t)B * 3 * (size_t)p->D * es;
    const size_t need = rglru_prefill_workspace_bytes(B, T, p->D, p->n_heads, p->dtype);
    if (!static_ws && T > 0 && (!workspace || ws_bytes < need)) return RGLRU_ERR_WORKSPACE;
    // outputs: out vs every input; state outputs may alias their own input exactly
    if (overlap(out, n_act, x, n_act) || overlap(out, n_act, y, n_act) ||
        overlap(out, n_act, h0, n_h) || overlap(out, n_act, h_last, n_h) ||
        overlap(out, n_act, conv0, n_c) || overlap(out, n_act, conv_last, n_c))
        return RGLRU_ERR_ALIAS;
    if (overlap(h_last, n_h, x, n_act) || overlap(h_last, n_h, y, n_act) ||
        overlap(h_last, n_h, conv0, n_c) || overlap(h_last, n_h, conv_last, n_c) ||
        ((const void*)h_last != (const void*)h0 && overlap(h_last, n_h, h0, n_h)))
        return RGLRU_ERR_ALIAS;
    if (overlap(conv_last, n_c, x, n_act) || overlap(conv_last, n_c, y, n_act) ||
        overlap(conv_last, n_c, h0, n_h) ||
        (conv_last != conv0 && overlap(conv_last, n_c, conv0, n_c)))
        return RGLRU_ERR_ALIAS;
    if (T > 0 && !static_ws) {
        const void* ins[] = {x, y, out, h0, h_last, conv0, conv_last};
        const size_t lens[] = {n_act, n_act, n_act, n_h, n_h, n_c, n_c};
        for (int i = 0; i < 7; ++i)
            if (overlap(workspace, need, ins[i], lens[i])) return RGLRU_ERR_ALIAS;
    }
    return RGLRU_OK;
}

}  // namespace

extern "C" {

int rglru_prefill(const rglru_params* p, int32_t B, int32_t T, const void* x, const void* y,
                  void* out, const float* h0, float* h_last, const void* conv0, void* conv_last,
                  void* workspace, size_t ws_bytes, void* stream) {
    const int st = check_prefill(p, B, T, x, y, out, h0, h_last, conv0, conv_last, workspace,
                                 ws_bytes);
    if (st != RGLRU_OK) return st;

    PrefillArgs a;
    memset(&a, 0, sizeof a);
    a.x = x; a.y = y; a.out = out;
    a.conv_w = p->conv_w; a.conv_b = p->conv_b;
    a.wa = p->gate_a_w; a.ba = p->gate_a_b; a.wx = p->gate_x_w; a.bx = p->gate_x_b;
    a.lambda = p->lambda;
    a.h0 = h0; a.h_last = h_last; a.conv0 = conv0; a.conv_last = conv_last;
    a.B = B; a.T = T; a.D = p->D; a.H = p->n_heads;
    hipError_t e;
    if (T == 0) {
        if (!h_last && !conv_last) return RGLRU_OK;
        e = launch_prefill_empty(a, p->dtype, (hipStream_t)stream);
        return e == hipSuccess ? RGLRU_OK : hip_fail(e);
    }
    const size_t S = n_segments(T);
    const size_t units = S * (size_t)B * (size_t)p->n_heads;
    if (units > 0x7fffffffu) return RGLRU_ERR_SHAPE;
    a.S = (int)S;
    a.n_units = (int)units;
    a.header = static_cast<unsigned*>(workspace);
    a.words = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + kWsHeader);
    e = launch_prefill(a, p->dtype, p->D / p->n_heads, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

}  // extern "C"

// ------------------------------------------------------------------------------------------
// Allocation-free prefill: the look-back state (header and carry words) lives in a static
// device array instead of a caller workspace.  Each GPU holds its own copy of the array until
// the process ends, and every call on a GPU shares it, so calls that overlap on one GPU race.
// In host code `scratch` only names the symbol: its device address on the current GPU is
// looked up once per device (hipGetSymbolAddress) and only that address reaches the kernels.
// Every call sets up the part it uses on its stream (header cleared, carry words "not
// ready"), so nothing depends on what an earlier call left there.
// ------------------------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = RGLRU_PREFILL_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device.
int scratch_address(void** addr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return RGLRU_ERR_UNSUPPORTED;
    void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        ptr = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e);
            if (ptr == nullptr) return hip_fail(hipErrorInvalidSymbol);
            g_scratch_addr[dev].store(ptr, std::memory_order_release);
        }
    }
    *addr = ptr;
    return RGLRU_OK;
}

}  // namespace

extern "C" {

int rglru_prefill_noalloc(const rglru_params* p, int32_t B, int32_t T, const void* x,
                          const void* y, void* out, const float* h0, float* h_last,
                          const void* conv0, void* conv_last, void* stream) {
    int st = check_prefill(p, B, T, x, y, out, h0, h_last, conv0, conv_last, nullptr, 0, true);
    if (st != RGLRU_OK) return st;
    const size_t need = rglru_prefill_workspace_bytes(B, T, p->D, p->n_heads, p->dtype);
    if (need > kScratchBytes) return RGLRU_ERR_WORKSPACE;
    void* ws = nullptr;
    if (T > 0) {
        st = scratch_address(&ws);
        if (st != RGLRU_OK) return st;
    }
    return rglru_prefill(p, B, T, x, y, out, h0, h_last, conv0, conv_last, ws,
                         T > 0 ? kScratchBytes : 0, stream);
}

size_t rglru_decode_workspace_bytes(int32_t N, int32_t D, int32_t dtype) {
    if (N < 1 || D < 1) return 0;
    return (size_t)((N + 15) / 16) * 16 * (size_t)D * elem_size(dtype);  // blocks of 16 sequences
}

// the decode step: every check runs first; with launch = false nothing else happens
static int decode_step_impl(const rglru_params* p, int32_t N, const void* x_t, int64_t ld_x,
                            const void* y_t, int64_t ld_y, void* out_t, int64_t ld_out, float* h,
                            void* conv_state, void* workspace, size_t ws_bytes, void* stream,
                            bool launch) {
    int st = check_params(p, true);
    if (st != RGLRU_OK) return st;
    if (N < 1) return RGLRU_ERR_SHAPE;
    if (!x_t || !y_t || !out_t || !h || !conv_state) return RGLRU_ERR_NULL;
    const int64_t D = p->D;
    if (ld_x == 0) ld_x = D;
    if (ld_y == 0) ld_y = D;
    if (ld_out == 0) ld_out = D;
    if (ld_x < D || ld_y < D || ld_out < D) return RGLRU_ERR_SHAPE;
    if (!aligned16(x_t) || !aligned16(y_t) || !aligned16(out_t) || !aligned16(h) ||
        !aligned16(conv_state))
        return RGLRU_ERR_UNSUPPORTED;
    const size_t es = elem_size(p->dtype);
    if ((ld_x * (int64_t)es) % 16 || (ld_y * (int64_t)es) % 16 || (ld_out * (int64_t)es) % 16)
        return RGLRU_ERR_UNSUPPORTED;
    const size_t sx = ((size_t)(N - 1) * (size_t)ld_x + (size_t)D) * es;
    const size_t sy = ((size_t)(N - 1) * (size_t)ld_y + (size_t)D) * es;
    const size_t so = ((size_t)(N - 1) * (size_t)ld_out + (size_t)D) * es;
    const size_t sh = (size_t)N * (size_t)D * sizeof(float);
    const size_t sc = (size_t)N * 3 * (size_t)D * es;
    if (overlap(out_t, so, x_t, sx) || overlap(out_t, so, y_t, sy) || overlap(out_t, so, h, sh) ||
        overlap(out_t, so, conv_state, sc) || overlap(h, sh, x_t, sx) || overlap(h, sh, y_t, sy) ||
        overlap(h, sh, conv_state, sc) || overlap(conv_state, sc, x_t, sx) ||
        overlap(conv_state, sc, y_t, sy))
        return RGLRU_ERR_ALIAS;
    if (workspace != nullptr) {
        const size_t need = rglru_decode_workspace_bytes(N, p->D, p->dtype);
        if (ws_bytes < need) return RGLRU_ERR_WORKSPACE;
        if (!aligned16(workspace)) return RGLRU_ERR_UNSUPPORTED;
        if (overlap(workspace, need, x_t, sx) || overlap(workspace, need, y_t, sy) ||
            overlap(workspace, need, out_t, so) || overlap(workspace, need, h, sh) ||
            overlap(workspace, need, conv_state, sc))
            return RGLRU_ERR_ALIAS;
    }
    if (!launch) return RGLRU_OK;
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.x = x_t; a.y = y_t; a.out = out_t;
    a.ld_x = ld_x; a.ld_y = ld_y; a.ld_out = ld_out;
    a.conv_w = p->conv_w; a.conv_b = p->conv_b;
    a.wa = p->gate_a_w; a.ba = p->gate_a_b; a.wx = p->gate_x_w; a.bx = p->gate_x_b;
    a.lambda = p->lambda;
    a.h = h; a.conv_state = conv_state;
    a.u_ws = workspace;
    a.N = N; a.D = p->D; a.H = p->n_heads;
    hipError_t e = launch_decode(a, p->dtype, p->D / p->n_heads, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

int rglru_decode_step(const rglru_params* p, int32_t N, const void* x_t, int64_t ld_x,
                      const void* y_t, int64_t ld_y, void* out_t, int64_t ld_out, float* h,
                      void* conv_state, void* workspace, size_t ws_bytes, void* stream) {
    return decode_step_impl(p, N, x_t, ld_x, y_t, ld_y, out_t, ld_out, h, conv_state, workspace,
                            ws_bytes, stream, true);
}

int conv1d_state_update(const rglru_params* p, int32_t N, int32_t T_new, const void* x_new,
                        void* conv_state, void* conv_out, void* stream) {
    int st = check_params(p, false);
    if (st != RGLRU_OK) return st;
    if (N < 1 || T_new < 0) return RGLRU_ERR_SHAPE;
    if (!conv_state || (T_new > 0 && !x_new)) return RGLRU_ERR_NULL;
    if (!aligned16(x_new) || !aligned16(conv_state) || !aligned16(conv_out))
        return RGLRU_ERR_UNSUPPORTED;
    const size_t es = elem_size(p->dtype);
    const size_t sx = (size_t)N * (size_t)T_new * (size_t)p->D * es;
    const size_t sc = (size_t)N * 3 * (size_t)p->D * es;
    if (overlap(conv_out, sx, x_new, sx) || overlap(conv_out, sx, conv_state, sc) ||
        overlap(conv_state, sc, x_new, sx))
        return RGLRU_ERR_ALIAS;
    if (T_new == 0) return RGLRU_OK;  // nothing to convolve; the window is unchanged
    ConvArgs a;
    a.x = x_new; a.conv_w = p->conv_w; a.conv_b = p->conv_b;
    a.conv_state = conv_state; a.conv_out = conv_out;
    a.N = N; a.T = T_new; a.D = p->D;
    hipError_t e = launch_conv_update(a, p->dtype, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

int rglru_linear(int32_t M, int32_t K, int32_t N, const void* x, const void* w, const void* b,
                 void* out, void* stream) {
    if (M < 0 || K < 1 || N < 1) return RGLRU_ERR_SHAPE;
    if (K % 128 != 0 || N % 256 != 0 || K >= (1 << 22) || N >= (1 << 22))
        return RGLRU_ERR_UNSUPPORTED;
    if (!w || (M > 0 && (!x || !out))) return RGLRU_ERR_NULL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(b) || !aligned16(out))
        return RGLRU_ERR_UNSUPPORTED;
    const size_t nx = (size_t)M * K * 2, no = (size_t)M * N * 2;
    if (overlap(out, no, x, nx) || overlap(out, no, w, (size_t)N * K * 2) ||
        overlap(out, no, b, (size_t)N * 2))
        return RGLRU_ERR_ALIAS;
    if (M == 0) return RGLRU_OK;
    ProjGemmArgs g;
    memset(&g, 0, sizeof g);
    g.A = x; g.W[0] = w; g.b[0] = b; g.C[0] = out;
    g.M = M; g.K = K; g.Nw[0] = N; g.nseg = 1;
    hipError_t e = launch_proj_gemm(g, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

size_t rglru_block_prefill_workspace_bytes(int32_t B, int32_t T, int32_t D, int32_t n_heads,
                                           int32_t D_model, int32_t dtype) {
    const size_t pw = rglru_prefill_workspace_bytes(B, T, D, n_heads, dtype);
    if (pw == 0 || D_model < 1) return 0;
    const size_t act = ((size_t)B * (size_t)T * (size_t)D * elem_size(dtype) + 255) & ~(size_t)255;
    return ((pw + 255) & ~(size_t)255) + 3 * act;
}

}  // extern "C"

namespace {

// The recurrent block: every check runs first; with launch = false nothing else happens.
int block_prefill_impl(const rglru_params* p, const rglru_proj_params* q, int32_t B, int32_t T,
                       const void* x_in, void* out, const float* h0, float* h_last,
                       const void* conv0, void* conv_last, void* workspace, size_t ws_bytes,
                       void* stream, bool launch) {
    int st = check_params(p, true);
    if (st != RGLRU_OK) return st;
    if (!q) return RGLRU_ERR_NULL;
    if (p->dtype != RGLRU_BF16) return RGLRU_ERR_UNSUPPORTED;
    if (B < 1 || T < 0 || q->D_model < 1) return RGLRU_ERR_SHAPE;
    const int D = p->D, Dm = q->D_model;
    if (D % 256 != 0 || Dm % 256 != 0 || D >= (1 << 21) || Dm >= (1 << 21))
        return RGLRU_ERR_UNSUPPORTED;
    if (!q->lin_x_w || !q->lin_y_w || !q->lin_out_w) return RGLRU_ERR_NULL;
    if (T > 0 && (!x_in || !out)) return RGLRU_ERR_NULL;
    const void* ptrs[] = {q->lin_x_w, q->lin_x_b, q->lin_y_w, q->lin_y_b, q->lin_out_w,
                          q->lin_out_b, x_in, out, workspace};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return RGLRU_ERR_UNSUPPORTED;
    if ((size_t)B * (size_t)T >= ((size_t)1 << 31)) return RGLRU_ERR_SHAPE;
    const size_t pw = rglru_prefill_workspace_bytes(B, T, D, p->n_heads, p->dtype);
    const size_t need = rglru_block_prefill_workspace_bytes(B, T, D, p->n_heads, Dm, p->dtype);
    if (T > 0 && (!workspace || ws_bytes < need)) return RGLRU_ERR_WORKSPACE;
    const size_t n_io = (size_t)B * T * Dm * 2;
    const size_t n_h = (size_t)B * D * sizeof(float), n_c = (size_t)B * 3 * D * 2;
    if (overlap(out, n_io, x_in, n_io) || overlap(out, n_io, h0, n_h) ||
        overlap(out, n_io, h_last, n_h) || overlap(out, n_io, conv0, n_c) ||
        overlap(out, n_io, conv_last, n_c))
        return RGLRU_ERR_ALIAS;
    if (T > 0) {
        const void* ins[] = {x_in, out, h0, h_last, conv0, conv_last, q->lin_x_w, q->lin_y_w,
                             q->lin_out_w};
        const size_t lens[] = {n_io, n_io, n_h, n_h, n_c, n_c, (size_t)D * Dm * 2,
                               (size_t)D * Dm * 2, (size_t)D * Dm * 2};
        for (int i = 0; i < 9; ++i)
            if (overlap(workspace, need, ins[i], lens[i])) return RGLRU_ERR_ALIAS;
    }
    const size_t act = ((size_t)B * T * D * 2 + 255) & ~(size_t)255;
    char* base = T > 0 ? static_cast<char*>(workspace) + ((pw + 255) & ~(size_t)255) : nullptr;
    void* xb = base;
    void* yb = T > 0 ? base + act : nullptr;
    void* mg = T > 0 ? base + 2 * act : nullptr;
    // the path's own checks, before anything is launched
    st = check_prefill(p, B, T, xb, yb, mg, h0, h_last, conv0, conv_last, workspace, pw);
    if (st != RGLRU_OK || !launch) return st;
    if (T == 0)  // state pass-through only
        return rglru_prefill(p, B, 0, nullptr, nullptr, nullptr, h0, h_last, conv0, conv_last,
                             nullptr, 0, stream);

    const int M = B * T;
    ProjGemmArgs g;
    memset(&g, 0, sizeof g);
    g.A = x_in; g.W[0] = q->lin_x_w; g.W[1] = q->lin_y_w; g.b[0] = q->lin_x_b; g.b[1] = q->lin_y_b;
    g.C[0] = xb; g.C[1] = yb; g.M = M; g.K = Dm; g.Nw[0] = D; g.Nw[1] = D; g.nseg = 2;
    hipError_t e = launch_proj_gemm(g, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    st = rglru_prefill(p, B, T, xb, yb, mg, h0, h_last, conv0, conv_last, workspace, pw, stream);
    if (st != RGLRU_OK) return st;
    memset(&g, 0, sizeof g);
    g.A = mg; g.W[0] = q->lin_out_w; g.b[0] = q->lin_out_b; g.C[0] = out;
    g.M = M; g.K = D; g.Nw[0] = Dm; g.nseg = 1;
    e = launch_proj_gemm(g, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int rglru_block_prefill(const rglru_params* p, const rglru_proj_params* q, int32_t B, int32_t T,
                        const void* x_in, void* out, const float* h0, float* h_last,
                        const void* conv0, void* conv_last, void* workspace, size_t ws_bytes,
                        void* stream) {
    return block_prefill_impl(p, q, B, T, x_in, out, h0, h_last, conv0, conv_last, workspace,
                              ws_bytes, stream, true);
}

// ------------------------------------------------------------------------------------------
// local sliding-window multi-query attention
// ------------------------------------------------------------------------------------------
size_t rglru_local_attention_workspace_bytes(int32_t B, int32_t T, int32_t n_heads) {
    if (B < 1 || T < 0 || n_heads < 1) return 0;
    const size_t M = (size_t)B * (size_t)T, T4 = ((size_t)T + 3) / 4;
    return round256(M * n_heads * kAttnDh * 2) + round256(M * kAttnDh * 2) +
           round256((size_t)B * T4 * kAttnDh * 4 * 2);
}

size_t rglru_local_attention_cache_bytes(int32_t N, int32_t window) {
    if (N < 1 || window < 1 || window >= (1 << 22)) return 0;
    return (size_t)N * (size_t)((window + 31) / 32) * 32 * kAttnDh * 2;
}

int rglru_local_attention(int32_t B, int32_t T, int32_t n_heads, int32_t window, float rope_base,
                          const void* q, const void* k, const void* v, void* o, void* kcache,
                          void* vcache, void* workspace, size_t ws_bytes, void* stream) {
    if (B < 1 || T < 0 || n_heads < 1 || n_heads > 64 || window < 1 || !(rope_base > 1.0f) ||
        !(rope_base < INFINITY))
        return RGLRU_ERR_SHAPE;
    const long long T4 = ((long long)T + 3) / 4;
    if (T >= (1 << 22) || (long long)B * 4 * T4 >= (1LL << 24) ||
        (long long)B * n_heads * (((long long)T + 127) / 128) >= (1LL << 24))
        return RGLRU_ERR_UNSUPPORTED;
    if (window >= (1 << 22)) return RGLRU_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !o)) return RGLRU_ERR_NULL;
    if ((kcache == nullptr) != (vcache == nullptr)) return RGLRU_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) ||
        !aligned16(kcache) || !aligned16(vcache))
        return RGLRU_ERR_UNSUPPORTED;
    const size_t M = (size_t)B * T;
    const size_t nq = M * n_heads * kAttnDh * 2, nk = M * kAttnDh * 2;
    const size_t nc = kcache ? rglru_local_attention_cache_bytes(B, window) : 0;
    const size_t need = rglru_local_attention_workspace_bytes(B, T, n_heads);
    if (T > 0 && (!workspace || ws_bytes < need)) return RGLRU_ERR_WORKSPACE;
    const void* outs[] = {o, kcache, vcache};
    const size_t outn[] = {nq, nc, nc};
    const void* ins[] = {q, k, v};
    const size_t inn[] = {nq, nk, nk};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j)
            if (overlap(outs[i], outn[i], ins[j], inn[j])) return RGLRU_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outn[i], outs[j], outn[j])) return RGLRU_ERR_ALIAS;
    }
    if (T > 0)
        for (int i = 0; i < 3; ++i)
            if (overlap(workspace, need, outs[i], outn[i]) || overlap(workspace, need, ins[i], inn[i]))
                return RGLRU_ERR_ALIAS;
    if (T == 0) return RGLRU_OK;
    AttnArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.kc = kcache; a.vc = vcache;
    a.Wc = (window + 31) / 32 * 32;
    char* ws = static_cast<char*>(workspace);
    a.qr = ws;
    a.kr = ws + round256(nq);
    a.v4 = ws + round256(nq) + round256(nk);
    a.B = B; a.T = T; a.Hq = n_heads; a.W = window; a.T4 = (int)T4; a.rope_base = rope_base;
    hipError_t e = launch_attention(a, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

size_t rglru_local_attention_decode_workspace_bytes(int32_t N, int32_t n_heads, int32_t window) {
    if (N < 1 || n_heads < 1 || window < 1 || window >= (1 << 22)) return 0;
    // the window splits per sequence shrink as the batch grows (attn_dec_tiles_per_wave), so the
    // size is taken as the largest over all batches up to N: a buffer sized for N fits any
    // smaller batch.  Within one split regime the size grows with N.
    size_t best = 0;
    const int32_t cand[3] = {N, std::min<int32_t>(N, 15), std::min<int32_t>(N, 63)};
    for (int32_t n : cand) {
        const size_t nsplit = (size_t)attn_dec_nsplit(n, window);
        best = std::max(best, round256((size_t)n * n_heads * kAttnDh * 2) +
                                  (size_t)n * nsplit * n_heads * (2 + kAttnDh) * sizeof(float));
    }
    return best;
}

// the attention decode step: every check runs first; with launch = false nothing else happens
static int attn_decode_impl(int32_t N, int32_t n_heads, int32_t window, float rope_base,
                            const int32_t* pos, const void* q, const void* k, const void* v,
                            void* kcache, void* vcache, void* o, void* workspace, size_t ws_bytes,
                            void* stream, bool launch) {
    if (N < 1 || n_heads < 1 || n_heads > 16 || window < 1 || !(rope_base > 1.0f) ||
        !(rope_base < INFINITY))
        return RGLRU_ERR_SHAPE;
    const long long nsplit = attn_dec_nsplit(N, window);
    if (window >= (1 << 22) || (long long)N * nsplit >= (1LL << 24)) return RGLRU_ERR_UNSUPPORTED;
    if (!pos || !q || !k || !v || !kcache || !vcache || !o) return RGLRU_ERR_NULL;
    const void* ptrs[] = {pos, q, k, v, kcache, vcache, o, workspace};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return RGLRU_ERR_UNSUPPORTED;
    const size_t need = rglru_local_attention_decode_workspace_bytes(N, n_heads, window);
    if (!workspace || ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t nq = (size_t)N * n_heads * kAttnDh * 2, nk = (size_t)N * kAttnDh * 2;
    const size_t nc = rglru_local_attention_cache_bytes(N, window);
    const void* all[] = {kcache, vcache, o, workspace, pos, q, k, v};
    const size_t len[] = {nc, nc, nq, need, (size_t)N * 4, nq, nk, nk};
    // the four written buffers overlap nothing; the read-only inputs may overlap each other
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 8; ++j)
            if (overlap(all[i], len[i], all[j], len[j])) return RGLRU_ERR_ALIAS;
    if (!launch) return RGLRU_OK;
    AttnDecodeArgs a;
    a.pos = pos; a.q = q; a.k = k; a.v = v; a.kc = kcache; a.vc = vcache; a.o = o;
    a.qr = workspace;
    a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      round256((size_t)N * n_heads * kAttnDh * 2));
    a.N = N; a.Hq = n_heads; a.W = window; a.Wc = (window + 31) / 32 * 32; a.nsplit = (int)nsplit;
    a.tpw = attn_dec_tiles_per_wave(N);
    a.rope_base = rope_base;
    hipError_t e = launch_attention_decode(a, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

int rglru_local_attention_decode(int32_t N, int32_t n_heads, int32_t window, float rope_base,
                                 const int32_t* pos, const void* q, const void* k, const void* v,
                                 void* kcache, void* vcache, void* o, void* workspace,
                                 size_t ws_bytes, void* stream) {
    return attn_decode_impl(N, n_heads, window, rope_base, pos, q, k, v, kcache, vcache, o,
                            workspace, ws_bytes, stream, true);
}

size_t rglru_local_attention_block_workspace_bytes(const rglru_attn_params* a, int32_t B,
                                                   int32_t T) {
    if (!a || B < 1 || T < 0 || a->n_heads < 1) return 0;
    const size_t M = (size_t)B * (size_t)T;
    const size_t nq = round256(M * a->n_heads * kAttnDh * 2), nk = round256(M * kAttnDh * 2);
    // q, k, v (projections), the attention output, then the attention's own workspace
    return 2 * nq + 2 * nk + rglru_local_attention_workspace_bytes(B, T, a->n_heads);
}

}  // extern "C"

namespace {

// The local-attention block (optionally filling the ring caches): every check runs first; with
// launch = false nothing else happens.
int attn_block_impl(const rglru_attn_params* a, int32_t B, int32_t T, const void* x_in, void* out,
                    void* kcache, void* vcache, void* workspace, size_t ws_bytes, void* stream,
                    bool launch) {
    if (!a) return RGLRU_ERR_NULL;
    if (a->head_dim != kAttnDh) return RGLRU_ERR_UNSUPPORTED;
    if (B < 1 || T < 0 || a->D_model < 1 || a->n_heads < 1 || a->n_heads > 64 || a->window < 1 ||
        !(a->rope_base > 1.0f) || !(a->rope_base < INFINITY))
        return RGLRU_ERR_SHAPE;
    const int Dm = a->D_model, Hq = a->n_heads;
    if (Dm % 256 != 0 || Dm >= (1 << 21)) return RGLRU_ERR_UNSUPPORTED;
    if (!a->q_w || !a->k_w || !a->v_w || !a->o_w) return RGLRU_ERR_NULL;
    if (T > 0 && (!x_in || !out)) return RGLRU_ERR_NULL;
    const void* ptrs[] = {a->q_w, a->k_w, a->v_w, a->o_w, a->o_b, x_in, out, workspace};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return RGLRU_ERR_UNSUPPORTED;
    const size_t M = (size_t)B * T;
    const size_t need = rglru_local_attention_block_workspace_bytes(a, B, T);
    if (T > 0 && (!workspace || ws_bytes < need)) return RGLRU_ERR_WORKSPACE;
    const size_t n_io = M * Dm * 2, HD = (size_t)Hq * kAttnDh;
    const size_t ins_len[] = {n_io, HD * Dm * 2, (size_t)kAttnDh * Dm * 2,
                              (size_t)kAttnDh * Dm * 2, HD * Dm * 2, (size_t)Dm * 2};
    const void* ins[] = {x_in, a->q_w, a->k_w, a->v_w, a->o_w, a->o_b};
    for (int i = 0; i < 6; ++i)
        if (overlap(out, n_io, ins[i], ins_len[i])) return RGLRU_ERR_ALIAS;
    if (T > 0) {
        if (overlap(workspace, need, out, n_io)) return RGLRU_ERR_ALIAS;
        for (int i = 0; i < 6; ++i)
            if (overlap(workspace, need, ins[i], ins_len[i])) return RGLRU_ERR_ALIAS;
    }
    const size_t nq = round256(M * HD * 2), nk = round256(M * kAttnDh * 2);
    char* ws = static_cast<char*>(workspace);
    void* qb = T > 0 ? ws : nullptr;
    void* kb = T > 0 ? ws + nq : nullptr;
    void* vb = T > 0 ? ws + nq + nk : nullptr;
    void* ob = T > 0 ? ws + nq + 2 * nk : nullptr;
    void* aw = T > 0 ? ws + 2 * nq + 2 * nk : nullptr;
    const size_t aw_bytes = rglru_local_attention_workspace_bytes(B, T, Hq);
    // the attention's own checks, before anything is launched
    int st = rglru_local_attention(B, 0, Hq, a->window, a->rope_base, qb, kb, vb, ob, kcache,
                                   vcache, aw, aw_bytes, stream);
    if (st != RGLRU_OK) return st;
    const long long T4 = ((long long)T + 3) / 4;
    if (T >= (1 << 22) || (long long)B * 4 * T4 >= (1LL << 24) ||
        (long long)B * Hq * (((long long)T + 127) / 128) >= (1LL << 24) ||
        M >= ((size_t)1 << 31))
        return RGLRU_ERR_UNSUPPORTED;
    if (kcache) {
        const size_t nc = rglru_local_attention_cache_bytes(B, a->window);
        if (overlap(kcache, nc, x_in, n_io) || overlap(vcache, nc, x_in, n_io) ||
            overlap(kcache, nc, out, n_io) || overlap(vcache, nc, out, n_io) ||
            (T > 0 && (overlap(kcache, nc, workspace, need) || overlap(vcache, nc, workspace, need))))
            return RGLRU_ERR_ALIAS;
        for (int i = 1; i < 6; ++i)
            if (overlap(kcache, nc, ins[i], ins_len[i]) || overlap(vcache, nc, ins[i], ins_len[i]))
                return RGLRU_ERR_ALIAS;
    }
    if (T == 0 || !launch) return RGLRU_OK;

    ProjGemmArgs g;
    memset(&g, 0, sizeof g);
    g.A = x_in; g.W[0] = a->q_w; g.W[1] = a->k_w; g.W[2] = a->v_w;
    g.C[0] = qb; g.C[1] = kb; g.C[2] = vb;
    g.M = (int)M; g.K = Dm; g.Nw[0] = (int)HD; g.Nw[1] = kAttnDh; g.Nw[2] = kAttnDh; g.nseg = 3;
    hipError_t e = launch_proj_gemm(g, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    st = rglru_local_attention(B, T, Hq, a->window, a->rope_base, qb, kb, vb, ob, kcache, vcache,
                               aw, aw_bytes, stream);
    if (st != RGLRU_OK) return st;
    memset(&g, 0, sizeof g);
    g.A = ob; g.W[0] = a->o_w; g.b[0] = a->o_b; g.C[0] = out;
    g.M = (int)M; g.K = (int)HD; g.Nw[0] = Dm; g.nseg = 1;
    e = launch_proj_gemm(g, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int rglru_local_attention_block(const rglru_attn_params* a, int32_t B, int32_t T,
                                const void* x_in, void* out, void* workspace, size_t ws_bytes,
                                void* stream) {
    return attn_block_impl(a, B, T, x_in, out, nullptr, nullptr, workspace, ws_bytes, stream, true);
}

int rglru_prefill_workspace_flags(void* workspace, size_t ws_bytes, uint32_t* flags_out,
                                  void* stream) {
    if (!workspace || !flags_out) return RGLRU_ERR_NULL;
    if (ws_bytes < kWsHeader) return RGLRU_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint32_t* hdr = static_cast<uint32_t*>(workspace);
    static const uint32_t zero = 0;
    hipError_t e = hipMemcpyAsync(flags_out, hdr + kErrWord, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipMemcpyAsync(hdr + kErrWord, &zero, sizeof(uint32_t), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

// ------------------------------------------------------------------------------------------
// the residual layer: RMSNorm, MLP, and the two layers
// ------------------------------------------------------------------------------------------
int rglru_rmsnorm(int32_t M, int32_t D, const void* x, const void* residual, const void* scale,
                  float eps, void* h_out, void* out, void* stream) {
    if (M < 0 || D < 1 || !(eps >= 0.0f) || !(eps < INFINITY)) return RGLRU_ERR_SHAPE;
    if (D % 8 != 0 || D > 8192 || (size_t)M * D >= ((size_t)1 << 40)) return RGLRU_ERR_UNSUPPORTED;
    if (M > 0 && (!x || (!h_out && !out) || (out && !scale))) return RGLRU_ERR_NULL;
    const void* ptrs[] = {x, residual, scale, h_out, out};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return RGLRU_ERR_UNSUPPORTED;
    const size_t n = (size_t)M * D * 2;
    if (overlap(out, n, x, n) || overlap(out, n, residual, n) || overlap(out, n, scale, D * 2) ||
        overlap(out, n, h_out, n) || overlap(h_out, n, residual, n) ||
        overlap(h_out, n, scale, D * 2) || (h_out != x && overlap(h_out, n, x, n)))
        return RGLRU_ERR_ALIAS;
    if (M == 0) return RGLRU_OK;
    NormArgs a;
    a.x = x; a.y = residual; a.g = scale; a.h = h_out; a.n = out; a.M = M; a.D = D; a.eps = eps;
    hipError_t e = launch_add_rmsnorm(a, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

size_t rglru_mlp_workspace_bytes(int32_t M, int32_t F) {
    if (M < 0 || F < 1) return 0;
    return 2 * round256((size_t)M * F * 2);
}

}  // extern "C"

namespace {

int check_mlp(const rglru_mlp_params* m, int Dm) {
    if (!m) return RGLRU_ERR_NULL;
    if (m->D_model != Dm || m->F < 1) return RGLRU_ERR_SHAPE;
    if (m->F % 256 != 0 || m->F >= (1 << 21) || Dm % 256 != 0 || Dm >= (1 << 21))
        return RGLRU_ERR_UNSUPPORTED;
    if (!m->gate_w || !m->up_w || !m->down_w) return RGLRU_ERR_NULL;
    const void* ptrs[] = {m->gate_w, m->gate_b, m->up_w, m->up_b, m->down_w, m->down_b};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return RGLRU_ERR_UNSUPPORTED;
    return RGLRU_OK;
}

// the MLP's read-only operands, for overlap checks
int mlp_operands(const rglru_mlp_params* m, const void** ptrs, size_t* lens) {
    const size_t w = (size_t)m->F * m->D_model * 2;
    const void* p[] = {m->gate_w, m->gate_b, m->up_w, m->up_b, m->down_w, m->down_b};
    const size_t l[] = {w, (size_t)m->F * 2, w, (size_t)m->F * 2, w, (size_t)m->D_model * 2};
    for (int i = 0; i < 6; ++i) {
        ptrs[i] = p[i];
        lens[i] = l[i];
    }
    return 6;
}

int check_norms(const rglru_norm_params* n, int Dm) {
    if (!n) return RGLRU_ERR_NULL;
    if (!n->temporal_scale || !n->channel_scale) return RGLRU_ERR_NULL;
    if (!(n->eps >= 0.0f) || !(n->eps < INFINITY)) return RGLRU_ERR_SHAPE;
    if (!aligned16(n->temporal_scale) || !aligned16(n->channel_scale) || Dm > 8192)
        return RGLRU_ERR_UNSUPPORTED;
    return RGLRU_OK;
}

// The MLP on M rows.  With the row kernel (one to four rows) and the mid-size tiles (65 to
// 1024 rows) the gating runs in the gate|up launch's epilogue or split reduction; a residual,
// when given, is added in the down launch's epilogue (row kernel) or row-wise sum
// (rows_epilogue) (*res_added tells the caller which happened).  With in_norm_g (row kernel
// only) x is the residual stream and the gate|up launch applies the RMSNorm before the MLP.
hipError_t run_mlp(const rglru_mlp_params* m, int M, const void* x, void* out, void* ws,
                   float* part, size_t part_bytes, hipStream_t s,
                   const void* residual = nullptr, bool* res_added = nullptr,
                   bool rows_epilogue = false, const void* in_norm_g = nullptr,
                   float in_norm_eps = 0.0f) {
    const size_t nf = (size_t)M * m->F;
    void* G = ws;
    void* U = static_cast<char*>(ws) + round256(nf * 2);
    const bool gated = proj_gemm_gated_ok(M, m->D_model);
    ProjGemmArgs g;
    memset(&g, 0, sizeof g);
    g.A = x; g.W[0] = m->gate_w; g.W[1] = m->up_w; g.b[0] = m->gate_b; g.b[1] = m->up_b;
    g.C[0] = G; g.C[1] = U; g.M = M; g.K = m->D_model; g.Nw[0] = m->F; g.Nw[1] = m->F; g.nseg = 2;
    g.part = part; g.part_bytes = part_bytes; g.gated = gated;
    g.in_norm_g = in_norm_g; g.in_norm_eps = in_norm_eps;
    hipError_t e = launch_proj_gemm(g, s);
    if (e == hipSuccess && !gated) e = launch_geglu(G, U, nf, s);
    if (e != hipSuccess) return e;
    // the final residual addition rides on the down projection: in the row kernel's epilogue,
    // or in the row-wise sum of its partials
    const bool fuse = residual && rows_epilogue && part;
    const bool add = residual && (proj_gemm_rows(M, m->F) || fuse);
    if (res_added) *res_added = add;
    memset(&g, 0, sizeof g);
    g.A = G; g.W[0] = m->down_w; g.b[0] = m->down_b; g.C[0] = out;
    g.M = M; g.K = m->F; g.Nw[0] = m->D_model; g.nseg = 1;
    g.part = part; g.part_bytes = part_bytes; g.R = add ? residual : nullptr;
    g.rows_epilogue = fuse;
    return launch_proj_gemm(g, s);
}

// Layer workspace after the block's own part: xn / hn, the block output / the MLP output, h,
// then the MLP's workspace.
// Decode layers add fp32 partial sums for the GEMMs' split K at the end.
struct LayerBufs {
    void *a, *b, *h, *mlp;
    float* part;
    size_t part_bytes;
};
LayerBufs layer_bufs(void* workspace, size_t block_bytes, size_t M, int Dm) {
    const size_t act = round256(M * Dm * 2);
    char* base = static_cast<char*>(workspace) + round256(block_bytes);
    return {base, base + act, base + 2 * act, base + 3 * act, nullptr, 0};
}
// Split-K partial bytes of the decode-time projections (M rows; N and K per GEMM), the
// largest over all row counts up to M (a buffer sized for M then fits any smaller batch): the
// split count changes only when the number of row tiles (128 or 256 rows) does, and within one
// tile count the bytes grow with the rows, so the largest value is at M or at a multiple of 128
// below it.
size_t decode_part_bytes(int M, const int (*nk)[2], int n, const int (*nk_rows)[2] = nullptr,
                         int n_rows = 0) {
    size_t b = 0;
    for (int m = std::min(M, 128);; m = std::min(m + 128, M)) {
        for (int i = 0; i < n; ++i) b = std::max(b, proj_gemm_part_bytes(m, nk[i][0], nk[i][1]));
        // the GEMMs whose sums carry the layer's add-and-norm (partials even without a split)
        for (int i = 0; i < n_rows; ++i)
            b = std::max(b, proj_gemm_part_bytes_rows_epilogue(m, nk_rows[i][0], nk_rows[i][1]));
        if (m >= M) break;
    }
    return round256(b);
}
size_t layer_tail_bytes(size_t M, int Dm, int F) {
    return 3 * round256(M * Dm * 2) + rglru_mlp_workspace_bytes((int32_t)M, F);
}

// Launches of the layer after validation: norm 1, the block (through `block`), h and norm 2,
// the MLP into out, the final residual addition in place (done by the MLP's last launch when
// that takes the row kernel).
// With fuse (decode layers of more than four rows, which have partial-sum space), the block's
// output projection is expected to write h = x_in + its output and the second norm itself
// (rows_epilogue; see fuse_out_proj), and the final residual addition rides on the down
// projection's sum.
// With fold (decode layers of one sequence whose projections all take the row kernel), no
// norm runs on its own: the block's first projection is expected to normalise x_in on the way
// in (in_norm_g = the temporal scale), its output projection to write h = x_in + its output
// into L.h (R), and the MLP's gate|up projection normalises h on the way in.
template <class Block>
int run_layer(const rglru_norm_params* nrm, const rglru_mlp_params* m, size_t M, int Dm,
              const void* x_in, void* out, const LayerBufs& L, hipStream_t s, Block block,
              bool fuse = false, bool fold = false) {
    NormArgs na;
    na.x = x_in; na.y = nullptr; na.g = nrm->temporal_scale; na.h = nullptr; na.n = L.a;
    na.M = (int)M; na.D = Dm; na.eps = nrm->eps;
    hipError_t e = hipSuccess;
    if (!fold) e = launch_add_rmsnorm(na, s);
    if (e != hipSuccess) return hip_fail(e);
    int st = block();
    if (st != RGLRU_OK) return st;
    if (!fuse && !fold) {
        na.x = x_in; na.y = L.b; na.g = nrm->channel_scale; na.h = L.h; na.n = L.a;
        e = launch_add_rmsnorm(na, s);
    }
    bool added = false;
    if (e == hipSuccess && fold)
        e = run_mlp(m, (int)M, L.h, out, L.mlp, L.part, L.part_bytes, s, L.h, &added, false,
                    nrm->channel_scale, nrm->eps);
    else if (e == hipSuccess)
        e = run_mlp(m, (int)M, L.a, out, L.mlp, L.part, L.part_bytes, s, L.h, &added, fuse);
    if (e != hipSuccess) return hip_fail(e);
    if (added) return RGLRU_OK;
    na.x = L.h; na.y = out; na.g = nullptr; na.h = out; na.n = nullptr;
    e = launch_add_rmsnorm(na, s);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

// The block's output projection in a fused decode layer: C = h = x_in + the projection, and
// the second norm of h into L.a, from the row-wise sum of its partials.
void fuse_out_proj(ProjGemmArgs& g, const rglru_norm_params* nrm, const void* x_in,
                   const LayerBufs& L) {
    g.rows_epilogue = 1;
    g.R = x_in;
    g.C[0] = L.h;
    g.norm_g = nrm->channel_scale;
    g.norm_out = L.a;
    g.norm_eps = nrm->eps;
}

// A decode layer of one sequence folds both norms into its projections when every projection
// takes the row kernel: the block's first and output projections (K = Dm and K = Kout), the
// MLP's gate|up (K = Dm) and down (K = F) projections.  (Every wave of a normalising launch
// forms the normalised row itself: for one row that costs less than a launch of the norm
// kernel; for two or four rows it costs more.)
bool fold_norms(int N, int Dm, int Kout, int F) {
    return N == 1 && proj_gemm_rows(N, Dm) && proj_gemm_rows(N, Kout) && proj_gemm_rows(N, F);
}

// out and the workspace against everything else the layer reads or writes
int check_layer_alias(const void* x_in, void* out, size_t n_io, void* ws, size_t need,
                      const void* const* others, const size_t* olen, int nothers) {
    if (overlap(out, n_io, x_in, n_io) || overlap(out, n_io, ws, need) ||
        overlap(ws, need, x_in, n_io))
        return RGLRU_ERR_ALIAS;
    for (int i = 0; i < nothers; ++i)
        if (overlap(out, n_io, others[i], olen[i]) || overlap(ws, need, others[i], olen[i]))
            return RGLRU_ERR_ALIAS;
    return RGLRU_OK;
}

// written state buffers (h, conv windows, ring caches) against the layer's read-only weights
int check_state_alias(const void* const* wr, const size_t* wl, int nw, const void* const* rd,
                      const size_t* rl, int nr) {
    for (int i = 0; i < nw; ++i)
        for (int j = 0; j < nr; ++j)
            if (overlap(wr[i], wl[i], rd[j], rl[j])) return RGLRU_ERR_ALIAS;
    return RGLRU_OK;
}

}  // namespace

extern "C" {

int rglru_mlp(const rglru_mlp_params* m, int32_t M, const void* x, void* out, void* workspace,
              size_t ws_bytes, void* stream) {
    if (!m) return RGLRU_ERR_NULL;
    int st = check_mlp(m, m->D_model);
    if (st != RGLRU_OK) return st;
    if (M < 0) return RGLRU_ERR_SHAPE;
    if (M > 0 && (!x || !out)) return RGLRU_ERR_NULL;
    if (!aligned16(x) || !aligned16(out) || !aligned16(workspace)) return RGLRU_ERR_UNSUPPORTED;
    const size_t need = rglru_mlp_workspace_bytes(M, m->F);
    if (M > 0 && (!workspace || ws_bytes < need)) return RGLRU_ERR_WORKSPACE;
    const size_t n_io = (size_t)M * m->D_model * 2;
    const void* w[6];
    size_t wl[6];
    mlp_operands(m, w, wl);
    if (M > 0 && check_layer_alias(x, out, n_io, workspace, need, w, wl, 6) != RGLRU_OK)
        return RGLRU_ERR_ALIAS;
    if (M == 0) return RGLRU_OK;
    hipError_t e = run_mlp(m, M, x, out, workspace, nullptr, 0, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

size_t rglru_recurrent_layer_workspace_bytes(int32_t B, int32_t T, int32_t D, int32_t n_heads,
                                             int32_t D_model, int32_t F) {
    const size_t bw = rglru_block_prefill_workspace_bytes(B, T, D, n_heads, D_model, RGLRU_BF16);
    if (bw == 0 || F < 1) return 0;
    return round256(bw) + layer_tail_bytes((size_t)B * T, D_model, F);
}

int rglru_recurrent_layer_prefill(const rglru_params* p, const rglru_proj_params* q,
                                  const rglru_norm_params* nrm, const rglru_mlp_params* m,
                                  int32_t B, int32_t T, const void* x_in, void* out,
                                  const float* h0, float* h_last, const void* conv0,
                                  void* conv_last, void* workspace, size_t ws_bytes,
                                  void* stream) {
    if (!p || !q) return RGLRU_ERR_NULL;
    const int Dm = q->D_model;
    int st = check_norms(nrm, Dm);
    if (st == RGLRU_OK) st = check_mlp(m, Dm);
    if (st != RGLRU_OK) return st;
    if (B < 1 || T < 0) return RGLRU_ERR_SHAPE;
    if (T > 0 && (!x_in || !out)) return RGLRU_ERR_NULL;
    if (!aligned16(x_in) || !aligned16(out) || !aligned16(workspace)) return RGLRU_ERR_UNSUPPORTED;
    const size_t M = (size_t)B * T;
    const size_t bw = rglru_block_prefill_workspace_bytes(B, T, p->D, p->n_heads, Dm, RGLRU_BF16);
    const size_t need = rglru_recurrent_layer_workspace_bytes(B, T, p->D, p->n_heads, Dm, m->F);
    if (T > 0 && (bw == 0 || need == 0)) return RGLRU_ERR_SHAPE;
    if (T > 0 && (!workspace || ws_bytes < need)) return RGLRU_ERR_WORKSPACE;
    const LayerBufs L = layer_bufs(workspace, bw, M, Dm);
    // the block's own checks on the buffers the layer hands it (nothing is launched yet)
    st = block_prefill_impl(p, q, B, T, T > 0 ? L.a : nullptr, T > 0 ? L.b : nullptr, h0, h_last,
                            conv0, conv_last, T > 0 ? workspace : nullptr, T > 0 ? bw : 0, stream,
                            false);
    if (st != RGLRU_OK) return st;
    if (T == 0)   // state pass-through only
        return block_prefill_impl(p, q, B, 0, nullptr, nullptr, h0, h_last, conv0, conv_last,
                                  nullptr, 0, stream, true);
    const size_t n_io = M * Dm * 2, n_h = (size_t)B * p->D * 4, n_c = (size_t)B * 3 * p->D * 2;
    const size_t pw = (size_t)p->D * Dm * 2;
    const void* others[16] = {h0, h_last, conv0, conv_last, nrm->temporal_scale,
                              nrm->channel_scale, q->lin_x_w, q->lin_y_w, q->lin_out_w};
    size_t olen[16] = {n_h, n_h, n_c, n_c, (size_t)Dm * 2, (size_t)Dm * 2, pw, pw, pw};
    const int n = 9 + mlp_operands(m, others + 9, olen + 9);
    if (check_layer_alias(x_in, out, n_io, workspace, need, others, olen, n) != RGLRU_OK ||
        check_state_alias(others + 1, olen + 1, 1, others + 4, olen + 4, n - 4) != RGLRU_OK ||
        check_state_alias(others + 3, olen + 3, 1, others + 4, olen + 4, n - 4) != RGLRU_OK)
        return RGLRU_ERR_ALIAS;
    return run_layer(nrm, m, M, Dm, x_in, out, L, (hipStream_t)stream, [&]() {
        return block_prefill_impl(p, q, B, T, L.a, L.b, h0, h_last, conv0, conv_last, workspace,
                                  bw, stream, true);
    });
}

size_t rglru_attention_layer_workspace_bytes(const rglru_attn_params* a, int32_t B, int32_t T,
                                             int32_t F) {
    const size_t bw = rglru_local_attention_block_workspace_bytes(a, B, T);
    if (bw == 0 || F < 1) return 0;
    return round256(bw) + layer_tail_bytes((size_t)B * T, a->D_model, F);
}

int rglru_attention_layer_prefill(const rglru_attn_params* a, const rglru_norm_params* nrm,
                                  const rglru_mlp_params* m, int32_t B, int32_t T,
                                  const void* x_in, void* out, void* kcache, void* vcache,
                                  void* workspace, size_t ws_bytes, void* stream) {
    if (!a) return RGLRU_ERR_NULL;
    const int Dm = a->D_model;
    int st = check_norms(nrm, Dm);
    if (st == RGLRU_OK) st = check_mlp(m, Dm);
    if (st != RGLRU_OK) return st;
    if (B < 1 || T < 0 || a->n_heads < 1) return RGLRU_ERR_SHAPE;
    if (T > 0 && (!x_in || !out)) return RGLRU_ERR_NULL;
    if (!aligned16(x_in) || !aligned16(out) || !aligned16(workspace)) return RGLRU_ERR_UNSUPPORTED;
    const size_t M = (size_t)B * T;
    const size_t bw = rglru_local_attention_block_workspace_bytes(a, B, T);
    const size_t need = rglru_attention_layer_workspace_bytes(a, B, T, m->F);
    if (T > 0 && (bw == 0 || need == 0)) return RGLRU_ERR_SHAPE;
    if (T > 0 && (!workspace || ws_bytes < need)) return RGLRU_ERR_WORKSPACE;
    const LayerBufs L = layer_bufs(workspace, bw, M, Dm);
    st = attn_block_impl(a, B, T, T > 0 ? L.a : nullptr, T > 0 ? L.b : nullptr, kcache, vcache,
                         T > 0 ? workspace : nullptr, T > 0 ? bw : 0, stream, false);
    if (st != RGLRU_OK || T == 0) return st;
    const size_t n_io = M * Dm * 2, HD = (size_t)a->n_heads * kAttnDh;
    const size_t nc = kcache ? rglru_local_attention_cache_bytes(B, a->window) : 0;
    const void* others[16] = {kcache, vcache, nrm->temporal_scale, nrm->channel_scale, a->q_w,
                              a->k_w, a->v_w, a->o_w, a->o_b};
    size_t olen[16] = {nc, nc, (size_t)Dm * 2, (size_t)Dm * 2, HD * Dm * 2,
                       (size_t)kAttnDh * Dm * 2, (size_t)kAttnDh * Dm * 2, HD * Dm * 2,
                       (size_t)Dm * 2};
    const int n = 9 + mlp_operands(m, others + 9, olen + 9);
    if (check_layer_alias(x_in, out, n_io, workspace, need, others, olen, n) != RGLRU_OK ||
        check_state_alias(others, olen, 2, others + 2, olen + 2, n - 2) != RGLRU_OK)
        return RGLRU_ERR_ALIAS;
    return run_layer(nrm, m, M, Dm, x_in, out, L, (hipStream_t)stream, [&]() {
        return attn_block_impl(a, B, T, L.a, L.b, kcache, vcache, workspace, bw, stream, true);
    });
}

// ------------------------------------------------------------------------------------------
// decode steps of the two layers
// ------------------------------------------------------------------------------------------
// block part of the recurrent decode workspace: x and y branches, their product, the decode
// step's own workspace
static size_t rec_dec_block_bytes(size_t N, int D) {
    return 3 * round256(N * D * 2) + round256(rglru_decode_workspace_bytes((int32_t)N, D,
                                                                           RGLRU_BF16));
}

static size_t rec_dec_part_bytes(int N, int D, int Dm, int F) {
    const int nk[4][2] = {{2 * D, Dm}, {Dm, D}, {2 * F, Dm}, {Dm, F}};
    const int nk_rows[2][2] = {{Dm, D}, {Dm, F}};   // output and down projections
    return decode_part_bytes(N, nk, 4, nk_rows, 2);
}

size_t rglru_recurrent_layer_decode_workspace_bytes(int32_t N, int32_t D, int32_t D_model,
                                                    int32_t F) {
    if (N < 1 || D < 1 || D_model < 1 || F < 1) return 0;
    return round256(rec_dec_block_bytes(N, D)) + layer_tail_bytes(N, D_model, F) +
           rec_dec_part_bytes(N, D, D_model, F);
}

int rglru_recurrent_layer_decode(const rglru_params* p, const rglru_proj_params* q,
                                 const rglru_norm_params* nrm, const rglru_mlp_params* m,
                                 int32_t N, const void* x_t, void* out_t, float* h,
                                 void* conv_state, void* workspace, size_t ws_bytes,
                                 void* stream) {
    int st = check_params(p, true);
    if (st != RGLRU_OK) return st;
    if (!q) return RGLRU_ERR_NULL;
    const int Dm = q->D_model, D = p->D;
    st = check_norms(nrm, Dm);
    if (st == RGLRU_OK) st = check_mlp(m, Dm);
    if (st != RGLRU_OK) return st;
    if (p->dtype != RGLRU_BF16 || D % 256 != 0 || D >= (1 << 21)) return RGLRU_ERR_UNSUPPORTED;
    if (N < 1) return RGLRU_ERR_SHAPE;
    if (!q->lin_x_w || !q->lin_y_w || !q->lin_out_w || !x_t || !out_t) return RGLRU_ERR_NULL;
    const void* ptrs[] = {q->lin_x_w, q->lin_x_b, q->lin_y_w, q->lin_y_b, q->lin_out_w,
                          q->lin_out_b, x_t, out_t, workspace};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return RGLRU_ERR_UNSUPPORTED;
    const size_t need = rglru_recurrent_layer_decode_workspace_bytes(N, D, Dm, m->F);
    if (!workspace || ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t bb = rec_dec_block_bytes(N, D), act = round256((size_t)N * D * 2);
    char* ws = static_cast<char*>(workspace);
    void *xb = ws, *yb = ws + act, *mg = ws + 2 * act, *dws = ws + 3 * act;
    const size_t dws_bytes = rglru_decode_workspace_bytes(N, D, RGLRU_BF16);
    st = decode_step_impl(p, N, xb, D, yb, D, mg, D, h, conv_state, dws, dws_bytes, stream, false);
    if (st != RGLRU_OK) return st;
    const size_t n_io = (size_t)N * Dm * 2, pw = (size_t)D * Dm * 2;
    const void* others[16] = {h, conv_state, nrm->temporal_scale, nrm->channel_scale,
                              q->lin_x_w, q->lin_y_w, q->lin_out_w};
    size_t olen[16] = {(size_t)N * D * 4, (size_t)N * 3 * D * 2, (size_t)Dm * 2, (size_t)Dm * 2,
                       pw, pw, pw};
    const int n = 7 + mlp_operands(m, others + 7, olen + 7);
    if (check_layer_alias(x_t, out_t, n_io, workspace, need, others, olen, n) != RGLRU_OK ||
        check_state_alias(others, olen, 2, others + 2, olen + 2, n - 2) != RGLRU_OK)
        return RGLRU_ERR_ALIAS;
    LayerBufs L = layer_bufs(workspace, bb, N, Dm);
    L.part_bytes = rec_dec_part_bytes(N, D, Dm, m->F);
    L.part = L.part_bytes ? reinterpret_cast<float*>(ws + need - L.part_bytes) : nullptr;
    const hipStream_t s = (hipStream_t)stream;
    const bool fuse = L.part && proj_gemm_rows_epilogue_ok(N);
    const bool fold = !fuse && fold_norms(N, Dm, D, m->F);
    return run_layer(nrm, m, N, Dm, x_t, out_t, L, s, [&]() {
        ProjGemmArgs g;
        memset(&g, 0, sizeof g);
        g.A = fold ? x_t : L.a; g.W[0] = q->lin_x_w; g.W[1] = q->lin_y_w; g.b[0] = q->lin_x_b;
        g.b[1] = q->lin_y_b; g.C[0] = xb; g.C[1] = yb; g.M = N; g.K = Dm; g.Nw[0] = D;
        g.Nw[1] = D; g.nseg = 2; g.part = L.part; g.part_bytes = L.part_bytes;
        if (fold) { g.in_norm_g = nrm->temporal_scale; g.in_norm_eps = nrm->eps; }
        hipError_t e = launch_proj_gemm(g, s);
        if (e != hipSuccess) return hip_fail(e);
        int r = decode_step_impl(p, N, xb, D, yb, D, mg, D, h, conv_state, dws, dws_bytes, stream,
                                 true);
        if (r != RGLRU_OK) return r;
        memset(&g, 0, sizeof g);
        g.A = mg; g.W[0] = q->lin_out_w; g.b[0] = q->lin_out_b; g.C[0] = L.b;
        g.M = N; g.K = D; g.Nw[0] = Dm; g.nseg = 1; g.part = L.part; g.part_bytes = L.part_bytes;
        if (fuse) fuse_out_proj(g, nrm, x_t, L);
        if (fold) { g.R = x_t; g.C[0] = L.h; }
        e = launch_proj_gemm(g, s);
        return e == hipSuccess ? RGLRU_OK : hip_fail(e);
    }, fuse, fold);
}

// block part of the attention decode workspace: q, k, v, the attention output, the attention
// decode's own workspace
static size_t attn_dec_block_bytes(size_t N, int Hq, int W) {
    return 2 * round256(N * Hq * kAttnDh * 2) + 2 * round256(N * kAttnDh * 2) +
           round256(rglru_local_attention_decode_workspace_bytes((int32_t)N, Hq, W));
}

static size_t attn_dec_part_bytes(int N, int Hq, int Dm, int F) {
    const int HD = Hq * kAttnDh;
    const int nk[4][2] = {{HD + 2 * kAttnDh, Dm}, {Dm, HD}, {2 * F, Dm}, {Dm, F}};
    const int nk_rows[2][2] = {{Dm, HD}, {Dm, F}};  // output and down projections
    return decode_part_bytes(N, nk, 4, nk_rows, 2);
}

size_t rglru_attention_layer_decode_workspace_bytes(const rglru_attn_params* a, int32_t N,
                                                    int32_t F) {
    if (!a || N < 1 || F < 1 || a->n_heads < 1 || a->window < 1 || a->D_model < 1) return 0;
    if (rglru_local_attention_decode_workspace_bytes(N, a->n_heads, a->window) == 0) return 0;
    return round256(attn_dec_block_bytes(N, a->n_heads, a->window)) +
           layer_tail_bytes(N, a->D_model, F) + attn_dec_part_bytes(N, a->n_heads, a->D_model, F);
}

int rglru_attention_layer_decode(const rglru_attn_params* a, const rglru_norm_params* nrm,
                                 const rglru_mlp_params* m, int32_t N, const int32_t* pos,
                                 const void* x_t, void* out_t, void* kcache, void* vcache,
                                 void* workspace, size_t ws_bytes, void* stream) {
    if (!a) return RGLRU_ERR_NULL;
    const int Dm = a->D_model, Hq = a->n_heads;
    int st = check_norms(nrm, Dm);
    if (st == RGLRU_OK) st = check_mlp(m, Dm);
    if (st != RGLRU_OK) return st;
    if (a->head_dim != kAttnDh) return RGLRU_ERR_UNSUPPORTED;
    if (N < 1 || Hq < 1 || Hq > 16 || a->window < 1) return RGLRU_ERR_SHAPE;
    if (!a->q_w || !a->k_w || !a->v_w || !a->o_w || !x_t || !out_t) return RGLRU_ERR_NULL;
    const void* ptrs[] = {a->q_w, a->k_w, a->v_w, a->o_w, a->o_b, x_t, out_t, workspace};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return RGLRU_ERR_UNSUPPORTED;
    const size_t need = rglru_attention_layer_decode_workspace_bytes(a, N, m->F);
    if (need == 0) return RGLRU_ERR_SHAPE;
    if (!workspace || ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t HD = (size_t)Hq * kAttnDh;
    const size_t nq = round256((size_t)N * HD * 2), nk = round256((size_t)N * kAttnDh * 2);
    char* ws = static_cast<char*>(workspace);
    void *qb = ws, *kb = ws + nq, *vb = ws + nq + nk, *ob = ws + nq + 2 * nk;
    void* dws = ws + 2 * nq + 2 * nk;
    const size_t dws_bytes = rglru_local_attention_decode_workspace_bytes(N, Hq, a->window);
    st = attn_decode_impl(N, Hq, a->window, a->rope_base, pos, qb, kb, vb, kcache, vcache, ob, dws,
                          dws_bytes, stream, false);
    if (st != RGLRU_OK) return st;
    const size_t n_io = (size_t)N * Dm * 2;
    const size_t nc = rglru_local_attention_cache_bytes(N, a->window);
    const void* others[16] = {pos, kcache, vcache, nrm->temporal_scale, nrm->channel_scale,
                              a->q_w, a->k_w, a->v_w, a->o_w, a->o_b};
    size_t olen[16] = {(size_t)N * 4, nc, nc, (size_t)Dm * 2, (size_t)Dm * 2, HD * Dm * 2,
                       (size_t)kAttnDh * Dm * 2, (size_t)kAttnDh * Dm * 2, HD * Dm * 2,
                       (size_t)Dm * 2};
    const int n = 10 + mlp_operands(m, others + 10, olen + 10);
    if (check_layer_alias(x_t, out_t, n_io, workspace, need, others, olen, n) != RGLRU_OK ||
        check_state_alias(others + 1, olen + 1, 2, others + 3, olen + 3, n - 3) != RGLRU_OK)
        return RGLRU_ERR_ALIAS;
    LayerBufs L = layer_bufs(workspace, attn_dec_block_bytes(N, Hq, a->window), N, Dm);
    L.part_bytes = attn_dec_part_bytes(N, Hq, Dm, m->F);
    L.part = L.part_bytes ? reinterpret_cast<float*>(ws + need - L.part_bytes) : nullptr;
    const hipStream_t s = (hipStream_t)stream;
    const bool fuse = L.part && proj_gemm_rows_epilogue_ok(N);
    const bool fold = !fuse && fold_norms(N, Dm, (int)HD, m->F);
    return run_layer(nrm, m, N, Dm, x_t, out_t, L, s, [&]() {
        ProjGemmArgs g;
        memset(&g, 0, sizeof g);
        g.A = fold ? x_t : L.a; g.W[0] = a->q_w; g.W[1] = a->k_w; g.W[2] = a->v_w;
        g.C[0] = qb; g.C[1] = kb; g.C[2] = vb;
        g.M = N; g.K = Dm; g.Nw[0] = (int)HD; g.Nw[1] = kAttnDh; g.Nw[2] = kAttnDh; g.nseg = 3;
        g.part = L.part; g.part_bytes = L.part_bytes;
        if (fold) { g.in_norm_g = nrm->temporal_scale; g.in_norm_eps = nrm->eps; }
        hipError_t e = launch_proj_gemm(g, s);
        if (e != hipSuccess) return hip_fail(e);
        int r = attn_decode_impl(N, Hq, a->window, a->rope_base, pos, qb, kb, vb, kcache, vcache,
                                 ob, dws, dws_bytes, stream, true);
        if (r != RGLRU_OK) return r;
        memset(&g, 0, sizeof g);
        g.A = ob; g.W[0] = a->o_w; g.b[0] = a->o_b; g.C[0] = L.b;
        g.M = N; g.K = (int)HD; g.Nw[0] = Dm; g.nseg = 1;
        g.part = L.part; g.part_bytes = L.part_bytes;
        if (fuse) fuse_out_proj(g, nrm, x_t, L);
        if (fold) { g.R = x_t; g.C[0] = L.h; }
        e = launch_proj_gemm(g, s);
        return e == hipSuccess ? RGLRU_OK : hip_fail(e);
    }, fuse, fold);
}

// ------------------------------------------------------------------------------------------
// backward pass of the path
// ------------------------------------------------------------------------------------------
static bool backward_shape_ok(int32_t B, int32_t T, int32_t D, int32_t n_heads) {
    return B >= 1 && T >= 32 && n_heads >= 1 && D == 256 * n_heads && T % 32 == 0 &&
           ((long long)B * T) % 256 == 0 && (long long)B * T < (1LL << 22) &&
           (long long)B * (T / 32) * D < (1LL << 31);
}

size_t rglru_prefill_backward_workspace_bytes(int32_t B, int32_t T, int32_t D, int32_t n_heads) {
    if (!backward_shape_ok(B, T, D, n_heads)) return 0;
    return backward_workspace_bytes(B, T, D, n_heads);
}

int rglru_prefill_backward(const rglru_params* p, int32_t B, int32_t T, const void* x,
                           const void* y, const float* h0, const void* conv0, const void* dout,
                           const float* dh_last, void* dx, void* dy, float* dconv_w,
                           float* dconv_b, float* dwa, float* dba, float* dwx, float* dbx,
                           float* dlambda, float* dh0, float* dconv0, void* workspace,
                           size_t ws_bytes, void* stream) {
    int st = check_params(p, true);
    if (st != RGLRU_OK) return st;
    if (B < 1 || T < 0) return RGLRU_ERR_SHAPE;
    if (p->dtype != RGLRU_BF16 || !backward_shape_ok(B, T, p->D, p->n_heads))
        return RGLRU_ERR_UNSUPPORTED;
    const void* outs[] = {dx, dy, dconv_w, dconv_b, dwa, dba, dwx, dbx, dlambda, dh0, dconv0};
    if (!x || !y || !dout) return RGLRU_ERR_NULL;
    for (const void* o : outs)
        if (!o) return RGLRU_ERR_NULL;
    const void* ins[] = {x, y, h0, conv0, dout, dh_last, p->conv_w, p->conv_b, p->gate_a_w,
                         p->gate_a_b, p->gate_x_w, p->gate_x_b, p->lambda};
    for (const void* q : ins)
        if (!aligned16(q)) return RGLRU_ERR_UNSUPPORTED;
    for (const void* o : outs)
        if (!aligned16(o)) return RGLRU_ERR_UNSUPPORTED;
    if (!aligned16(workspace)) return RGLRU_ERR_UNSUPPORTED;
    const size_t need = rglru_prefill_backward_workspace_bytes(B, T, p->D, p->n_heads);
    if (!workspace || ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t D = p->D, H = p->n_heads, bs = D / H;
    const size_t act = (size_t)B * T * D * 2, st_b = (size_t)B * D * 4;
    const size_t olen[] = {act, act, D * 16, D * 4, H * bs * bs * 4, D * 4, H * bs * bs * 4, D * 4,
                           D * 4, st_b, (size_t)B * 3 * D * 4};
    const size_t ilen[] = {act, act, st_b, (size_t)B * 3 * D * 2, act, st_b, D * 8, D * 2,
                           H * bs * bs * 2, D * 2, H * bs * bs * 2, D * 2, D * 4};
    for (int i = 0; i < 11; ++i) {
        if (overlap(outs[i], olen[i], workspace, need)) return RGLRU_ERR_ALIAS;
        for (int j = i + 1; j < 11; ++j)
            if (overlap(outs[i], olen[i], outs[j], olen[j])) return RGLRU_ERR_ALIAS;
        for (int j = 0; j < 13; ++j)
            if (overlap(outs[i], olen[i], ins[j], ilen[j])) return RGLRU_ERR_ALIAS;
    }
    for (int j = 0; j < 13; ++j)
        if (overlap(workspace, need, ins[j], ilen[j])) return RGLRU_ERR_ALIAS;
    BwdArgs a;
    a.x = x; a.y = y; a.dout = dout; a.h0 = h0; a.conv0 = conv0; a.dh_last = dh_last;
    a.conv_w = p->conv_w; a.conv_b = p->conv_b; a.wa = p->gate_a_w; a.ba = p->gate_a_b;
    a.wx = p->gate_x_w; a.bx = p->gate_x_b; a.lambda = p->lambda;
    a.dx = dx; a.dy = dy; a.dconv_w = dconv_w; a.dconv_b = dconv_b; a.dwa = dwa; a.dba = dba;
    a.dwx = dwx; a.dbx = dbx; a.dlambda = dlambda; a.dh0 = dh0; a.dconv0 = dconv0;
    a.ws = workspace; a.B = B; a.T = T; a.D = (int)D; a.H = (int)H;
    hipError_t e = launch_prefill_backward(a, (hipStream_t)stream);
    return e == hipSuccess ? RGLRU_OK : hip_fail(e);
}

}  // extern "C"
