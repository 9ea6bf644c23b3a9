/*
 * rglru.h -- C ABI of the MI355X (gfx950) RG-LRU recurrent-block library (librglru.so).
 *
 * The operation is the recurrent block's temporal-mixing path of RecurrentGemma, as laid
 * out on the page "Gemma 詳解：RecurrentGemma 架構" (section "含遞迴區塊的殘差區塊" and the
 * module printout): two width-D branches; on one, a depthwise Conv1d with kernel 4
 * followed by the RG-LRU; on the other, GELU (tanh form); the branches are multiplied.
 * The library starts from the two branch projections' outputs:
 *
 *   x = linear_x(.), y = linear_y(.)            [B][T][D]  (inputs of every call)
 *   u_t   = conv_b + sum_{j=0..3} conv_w[:, j] * x_{t-3+j}     (causal, depthwise)
 *   r_t   = sigmoid(blockdiag(W_a) u_t + b_a),  i_t = sigmoid(blockdiag(W_x) u_t + b_x)
 *   a_t   = sigmoid(Lambda) ** (8 r_t)
 *   h_t   = a_t * h_{t-1} + sqrt(1 - a_t^2) * (i_t * u_t)
 *   out_t = h_t * gelu_tanh(y_t)
 *
 * The RG-LRU lines are the Griffin paper's definition (arXiv 2402.19427, linked from the
 * article "RecurrentGemma vs 传统LLM..."); the pages name the unit and its fixed-size
 * state ("模型寬度與 RNN 寬度") but print no formula.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; the rglru_params struct itself
 *     is host memory (read during the call only).
 *   - Tensors are row-major and contiguous with the channel axis D innermost.
 *   - The caller allocates and owns every buffer, including the prefill workspace.
 *   - Calls are asynchronous on the caller's HIP stream (passed as void*, NULL = default
 *     stream) and never synchronise the host.  Results are available after the stream
 *     reaches them.
 *   - Every call returns an rglru_status.  Arguments are validated on the host before any
 *     HIP call; a failing call leaves every buffer untouched.  RGLRU_ERR_HIP means a launch
 *     failed; the hipError_t is kept per thread (rglru_last_hip_error).  Faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - Results are deterministic: the same inputs give bitwise the same outputs (no float
 *     atomics; carries are always folded in sequence order).
 *   - Storage type `dtype` (RGLRU_F32 or RGLRU_BF16) applies to x, y, out, the conv state and
 *     all weights except Lambda; Lambda and the recurrent state h are always fp32.
 *   - Supported block sizes bs = D / n_heads: 128 and 256.  All pointers 16-byte aligned.
 */
#ifndef RGLRU_H
#define RGLRU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RGLRU_ABI_VERSION 7

enum rglru_dtype { RGLRU_F32 = 0, RGLRU_BF16 = 1 };

enum rglru_status {
    RGLRU_OK = 0,
    RGLRU_ERR_NULL = 1,        /* a required pointer is NULL */
    RGLRU_ERR_SHAPE = 2,       /* B/N < 1, T < 0, D < 1, n_heads < 1, D % n_heads != 0, bad stride */
    RGLRU_ERR_UNSUPPORTED = 3, /* bs not in {128, 256}, unknown dtype, pointer not 16-byte aligned,
                                  a bf16 prefill sequence (or conv window set) of 2 GiB or more,
                                  projection widths outside the multiples stated below */
    RGLRU_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than rglru_prefill_workspace_bytes */
    RGLRU_ERR_ALIAS = 5,       /* an output overlaps an input it may not alias */
    RGLRU_ERR_HIP = 6          /* a HIP call failed; see rglru_last_hip_error() */
};

/*
 * Parameters of one recurrent block (device pointers, storage type `dtype` unless noted).
 *   conv_w   [D][4]      tap j multiplies x_{t-3+j}: the first T outputs of PyTorch's
 *                        Conv1d(D, D, 4, padding=3, groups=D) weight [D][1][4], squeezed
 *   conv_b   [D] or NULL (NULL = no bias)
 *   gate_a_w [H][bs][bs] block h of the recurrence gate, stored like a Linear weight
 *                        [out j][in k]: pre_a[h*bs+j] = b_a[h*bs+j] + sum_k W_a[h][j][k] u[h*bs+k]
 *   gate_a_b [D] or NULL
 *   gate_x_w [H][bs][bs] input gate, same layout;  gate_x_b [D] or NULL
 *   lambda   [D] fp32    (always fp32)
 */
typedef struct rglru_params {
    int32_t D;
    int32_t n_heads;
    int32_t dtype;
    const void *conv_w;
    const void *conv_b;
    const void *gate_a_w;
    const void *gate_a_b;
    const void *gate_x_w;
    const void *gate_x_b;
    const float *lambda;
} rglru_params;

/*
 * Workspace management (no passage of the pages: these exist for the chunked scan's carries).
 * Bytes of device workspace rglru_prefill needs for this shape (0 on invalid shapes):
 * a 4096-byte header (error flags and ticket counters) and one 8-byte carry word per
 * (64-token segment except the last, sequence, channel).  The workspace needs no initialisation by the caller:
 * every prefill call first clears the header and sets the carry words it will use to "not
 * ready", on its own stream, with a fill kernel (no memset node, so the call may be captured
 * in a graph).  Any contents are therefore fine, including a fresh allocation or a buffer left
 * by a call of another shape.  The fill writes 8 * (ceil(T/64) - 1) * B * D bytes.
 * Calls sharing one workspace must be ordered on one stream (concurrent calls race).
 */
size_t rglru_prefill_workspace_bytes(int32_t B, int32_t T, int32_t D, int32_t n_heads,
                                     int32_t dtype);

/* Fills a whole workspace of ws_bytes bytes on `stream` (asynchronous): header zero, carry
 * words "not ready".  Never required (every prefill call prepares the part it uses); kept so
 * that callers of earlier versions of this header keep working. */
int rglru_prefill_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/*
 * Prefill over T tokens (the time-chunked scan).
 * Operation: the whole block path above over a prompt, page "Gemma 詳解：RecurrentGemma 架構",
 * section "含遞迴區塊的殘差區塊" (Conv1d -> RG-LRU branch times the GELU branch).
 *   x, y      [B][T][D]  inputs (storage dtype)
 *   out       [B][T][D]  h_t * gelu_tanh(y_t), rounded to the storage dtype (nearest-even)
 *   h0        [B][D] fp32 initial state, or NULL for zeros
 *   h_last    [B][D] fp32 state after token T-1, or NULL to skip
 *   conv0     [B][3][D]  last three conv inputs before token 0, oldest first, or NULL (zeros)
 *   conv_last [B][3][D]  last three conv inputs after the call, or NULL to skip
 *   workspace, ws_bytes  caller-owned device scratch (see above)
 * h0 == h_last and conv0 == conv_last (in place) are allowed; out must not overlap x or y.
 * T = 0 is valid: h_last = h0 and conv_last = conv0 (or zeros).
 * With bf16 storage one sequence must stay below 2 GiB (T * D * 2 < 2^31, e.g. T < 262144 at
 * D = 4096) and so must the conv windows of all B sequences (B * 3 * D * 2 < 2^31), else
 * RGLRU_ERR_UNSUPPORTED; longer sequences are prefilled in pieces, carrying h and the conv
 * window from one call to the next, and larger batches in several calls.
 */
int rglru_prefill(const rglru_params *p, int32_t B, int32_t T, const void *x, const void *y,
                  void *out, const float *h0, float *h_last, const void *conv0, void *conv_last,
                  void *workspace, size_t ws_bytes, void *stream);

/*
 * Prefill without a workspace argument, for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid allocation).  The same
 * operation, kernels and results as rglru_prefill (bitwise), with the look-back state in a
 * static device array of RGLRU_PREFILL_NOALLOC_MAX_BYTES bytes inside the library: every GPU
 * the library runs on holds one copy until the process ends.  The call allocates nothing.
 * A call whose rglru_prefill_workspace_bytes(B, T, D, n_heads, dtype) exceeds the maximum
 * returns RGLRU_ERR_WORKSPACE before any HIP call (the maximum covers B = 2, T = 65536,
 * D = 4096; longer inputs are prefilled in pieces, carrying h and the conv window).
 * All calls on one GPU share the array: calls that may overlap in time on one GPU (different
 * streams or threads) race and must be ordered by the caller.  The stream must belong to the
 * current device.  Other arguments and errors as for rglru_prefill.
 */
#define RGLRU_PREFILL_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int rglru_prefill_noalloc(const rglru_params *p, int32_t B, int32_t T, const void *x,
                          const void *y, void *out, const float *h0, float *h_last,
                          const void *conv0, void *conv_last, void *stream);

/*
 * Bytes of the optional decode workspace for N sequences: 16 * ceil(N / 16) * D storage
 * elements that hold the conv outputs u_t between the two passes of the split step, in blocks
 * of 16 sequences (16-byte aligned, contents need no initialisation and are not preserved
 * between calls).
 */
size_t rglru_decode_workspace_bytes(int32_t N, int32_t D, int32_t dtype);

/*
 * One decode step for N sequences (one token each), updating the carried state in place.
 * Operation: the same path for a single token, carrying the fixed-size state (h and the conv
 * window) that the page "Gemma 詳解：RecurrentGemma 架構" describes in sections
 * "模型寬度與 RNN 寬度" and "區域注意力視窗大小".
 *   x_t, y_t, out_t  [N][D] rows with element strides ld_x, ld_y, ld_out between rows
 *                    (0 means D), so a slice [:, t] of an [N][T][D] tensor needs no copy
 *   h                [N][D] fp32 state, read and written in place
 *   conv_state       [N][3][D] last three conv inputs, oldest first, read and written in place
 *   workspace, ws_bytes  NULL/0: one fused kernel per (32 sequences, gate head).  Otherwise a
 *                    device buffer of at least rglru_decode_workspace_bytes(N, D, dtype): with
 *                    bf16 storage the step runs as two kernels (conv pass into the workspace,
 *                    then a gate pass spread over 32-channel blocks), the faster form for
 *                    large N (up to N * D / 8 < 2^31; beyond that the fused kernel runs);
 *                    with fp32 storage the workspace is not used.  The two forms
 *                    leave identical conv windows; h and out agree to the rounding of the
 *                    fp32 gate sums, which the two forms accumulate in different orders.
 *                    The workspace must not overlap any other argument.
 * out_t must not overlap x_t, y_t, h or conv_state.
 */
int rglru_decode_step(const rglru_params *p, int32_t N, const void *x_t, int64_t ld_x,
                      const void *y_t, int64_t ld_y, void *out_t, int64_t ld_out, float *h,
                      void *conv_state, void *workspace, size_t ws_bytes, void *stream);

/*
 * Conv-state update (the conv part of the path on its own).
 *   x_new      [N][T_new][D] new conv inputs (storage dtype); T_new >= 0
 *   conv_state [N][3][D]     updated in place to the last three inputs, oldest first
 *   conv_out   [N][T_new][D] the conv outputs u_t (storage dtype, nearest-even), or NULL
 * Only p->D, p->dtype, p->conv_w and p->conv_b are read.  conv_out must not overlap x_new.
 */
/* Operation: the depthwise Conv1d (kernel 4, padding 3, groups D) of the module printout on the
 * page "Gemma 詳解：RecurrentGemma 架構", kept causal, and its three-token state. */
int conv1d_state_update(const rglru_params *p, int32_t N, int32_t T_new, const void *x_new,
                        void *conv_state, void *conv_out, void *stream);

/*
 * The dense projections around the path, which make it the whole temporal-mixing block.
 * Operation: the page "Gemma 詳解：RecurrentGemma 架構" (section "含遞迴區塊的殘差區塊" and the
 * module printout) applies two Linear layers with bias, linear_x and linear_y, to the block
 * input (width D_model) to form the two width-D branches, and a third, linear_out, to the
 * product of the branches, back to width D_model.  Weights are stored like PyTorch Linear
 * weights, [out][in].  bf16 storage only (operands bf16, fp32 accumulation, results rounded to
 * bf16 nearest-even).
 *   lin_x_w, lin_y_w  [D][D_model];  lin_x_b, lin_y_b  [D] or NULL (NULL = no bias)
 *   lin_out_w         [D_model][D];  lin_out_b         [D_model] or NULL
 */
typedef struct rglru_proj_params {
    int32_t D_model;
    const void *lin_x_w;
    const void *lin_x_b;
    const void *lin_y_w;
    const void *lin_y_b;
    const void *lin_out_w;
    const void *lin_out_b;
} rglru_proj_params;

/*
 * One Linear layer on its own: out[m][n] = b[n] + sum_k x[m][k] w[n][k] (bf16 storage).
 *   x [M][K], w [N][K] ([out][in]), b [N] or NULL, out [M][N]; M >= 0.
 * K % 128 == 0, N % 256 == 0, K < 2^22 and N < 2^22, else RGLRU_ERR_UNSUPPORTED.  out must not
 * overlap x, w or b.
 */
int rglru_linear(int32_t M, int32_t K, int32_t N, const void *x, const void *w, const void *b,
                 void *out, void *stream);

/*
 * Bytes of device workspace rglru_block_prefill needs: a prefill workspace (see
 * rglru_prefill_workspace_bytes) at offset 0, then room for the two branches and their
 * product ([B][T][D] each).  No initialisation is needed (the prefill part is prepared by every
 * call, as for rglru_prefill).  0 on invalid shapes.
 */
size_t rglru_block_prefill_workspace_bytes(int32_t B, int32_t T, int32_t D, int32_t n_heads,
                                           int32_t D_model, int32_t dtype);

/*
 * Prefill of the whole temporal-mixing block over T tokens:
 *   out = linear_out( path( linear_x(x_in), linear_y(x_in) ) )
 * where path is rglru_prefill's operation on the two branches.
 *   x_in  [B][T][D_model] block input;  out [B][T][D_model] block output (bf16)
 *   h0, h_last, conv0, conv_last  as for rglru_prefill (the conv window holds linear_x outputs)
 *   workspace, ws_bytes  at least rglru_block_prefill_workspace_bytes(...)
 * bf16 storage only; D % 256 == 0 and D_model % 256 == 0, else RGLRU_ERR_UNSUPPORTED (and the
 * limits of rglru_prefill apply).  out must not overlap x_in, the state buffers or the
 * workspace; the workspace must not overlap any other argument.
 */
int rglru_block_prefill(const rglru_params *p, const rglru_proj_params *q, int32_t B, int32_t T,
                        const void *x_in, void *out, const float *h0, float *h_last,
                        const void *conv0, void *conv_last, void *workspace, size_t ws_bytes,
                        void *stream);

/*
 * Local sliding-window multi-query attention, the model's other temporal-mixing block.
 * Operation: the page "Gemma 詳解：RecurrentGemma 架構" (section "含區域 MQA 的殘差區塊", the
 * module printout's RecurrentGemmaSdpaAttention, and section "區域注意力視窗大小") gives n_heads
 * query heads of width 256 sharing one key/value head, rotary position embedding on q and k,
 * and attention limited to a window of recent tokens.  Query t attends to tokens
 * max(0, t - window + 1) .. t of its own sequence:
 *   q', k'   = RoPE(q, t), RoPE(k, t): each pair (x_i, x_{i+128}) of a head is turned by the angle
 *              t * rope_base^(-2 i / 256), i = 0..127, positions t = 0..T-1 within each call
 *   o[t, h]  = sum_s softmax_s(q'[t, h] . k'[s] / 16) v[s]
 * bf16 storage only (fp32 scores and softmax, probabilities rounded to bf16 for the P.V
 * product, output rounded to bf16 nearest-even).
 *   q  [B][T][n_heads][256],  k, v  [B][T][256]   (before RoPE)
 *   o  [B][T][n_heads][256]
 *   kcache, vcache       optional ring caches for decoding (both or neither; NULL: not filled),
 *                        rglru_local_attention_cache_bytes(B, window) bytes each: the call writes
 *                        positions max(0, T - window) .. T-1 into them (see the decode step)
 *   workspace, ws_bytes  at least rglru_local_attention_workspace_bytes(B, T, n_heads); no
 *                        initialisation needed
 * B >= 1, T >= 0, 1 <= n_heads <= 64, window >= 1 and rope_base > 1, else RGLRU_ERR_SHAPE.
 * T < 2^22, B * 4 * ceil(T / 4) < 2^24 and B * n_heads * ceil(T / 128) < 2^24 (launch sizes),
 * else RGLRU_ERR_UNSUPPORTED.  o and the caches must not overlap q, k, v or each other; the
 * workspace must not overlap any other argument.  T = 0 launches nothing.
 */
size_t rglru_local_attention_workspace_bytes(int32_t B, int32_t T, int32_t n_heads);
int rglru_local_attention(int32_t B, int32_t T, int32_t n_heads, int32_t window, float rope_base,
                          const void *q, const void *k, const void *v, void *o, void *kcache,
                          void *vcache, void *workspace, size_t ws_bytes, void *stream);

/*
 * Ring KV cache of the local attention, for decoding: per sequence, Wc = 32 * ceil(window / 32)
 * slots of one key (after RoPE) and one value; slot t % window holds position t.  The slots are
 * grouped in tiles of 32 (16 KB of keys, 16 KB of values, bf16), each stored in the operand
 * order of the decode kernel's matrix instructions: within tile s / 32, slot r = s % 32 and
 * dimension d sit at element
 *   keys:    (((r / 16) * 8 + d / 32) * 4 + (d % 32) / 8) * 16 + r % 16) * 8 + d % 8
 *   values:  ((d / 16) * 4 + (r % 16) / 4) * 16 + d % 16) * 8 + r % 4 + 4 * (r / 16)
 * Bytes of one cache (keys or values) for N sequences; 0 on invalid arguments.  Slots that hold
 * no position of the current window are never read as values (their contents do not matter).
 */
size_t rglru_local_attention_cache_bytes(int32_t N, int32_t window);

/*
 * Decode step of the local attention: one new token for each of N sequences, at its own position.
 * Operation: as rglru_local_attention for the new token, which attends to positions
 * max(0, t - window + 1) .. t of its sequence, taken from the ring cache.
 *   pos               [N] int32 (device): the new token's position t >= 0 (a negative position
 *                     leaves that sequence's cache as it is and gives o = 0)
 *   q [N][n_heads][256], k, v [N][256]   the new token's q, k, v before RoPE
 *   kcache, vcache    rglru_local_attention_cache_bytes(N, window) bytes each, holding positions
 *                     max(0, t - window + 1) .. t - 1 (from rglru_local_attention or earlier
 *                     steps); the call writes position t into slot t % window
 *   o [N][n_heads][256]
 *   workspace, ws_bytes  at least rglru_local_attention_decode_workspace_bytes(N, n_heads,
 *                        window); no initialisation needed
 * N >= 1, 1 <= n_heads <= 16, window >= 1 and rope_base > 1, else RGLRU_ERR_SHAPE; window < 2^22
 * and N * ceil(window / S) < 2^24, else RGLRU_ERR_UNSUPPORTED, with S = 512 cache slots for
 * N >= 64, 256 for 16 <= N < 64 and 128 below.  No argument may overlap another (q, k and v
 * may overlap each other).  Deterministic: the window is split in fixed chunks of S slots whose
 * partial results are combined in chunk order.
 */
size_t rglru_local_attention_decode_workspace_bytes(int32_t N, int32_t n_heads, int32_t window);
int rglru_local_attention_decode(int32_t N, int32_t n_heads, int32_t window, float rope_base,
                                 const int32_t *pos, const void *q, const void *k, const void *v,
                                 void *kcache, void *vcache, void *o, void *workspace,
                                 size_t ws_bytes, void *stream);

/*
 * The whole local-attention block: the projections of the page's printout (q_proj, k_proj and
 * v_proj without bias, o_proj with bias) around rglru_local_attention:
 *   q = x_in q_w^T,  k = x_in k_w^T,  v = x_in v_w^T,  out = attention(q, k, v) o_w^T + o_b
 * Weights are stored like PyTorch Linear weights, [out][in], bf16:
 *   q_w [n_heads * 256][D_model],  k_w, v_w [256][D_model],  o_w [D_model][n_heads * 256],
 *   o_b [D_model] or NULL.
 * head_dim must be 256 and D_model % 256 == 0, else RGLRU_ERR_UNSUPPORTED; the limits of
 * rglru_local_attention apply.
 *   x_in, out  [B][T][D_model];  out must not overlap x_in, the weights or the workspace
 *   workspace, ws_bytes  at least rglru_local_attention_block_workspace_bytes(...)
 */
typedef struct rglru_attn_params {
    int32_t D_model;
    int32_t n_heads;
    int32_t head_dim;
    int32_t window;
    float rope_base;
    const void *q_w;
    const void *k_w;
    const void *v_w;
    const void *o_w;
    const void *o_b;
} rglru_attn_params;

size_t rglru_local_attention_block_workspace_bytes(const rglru_attn_params *a, int32_t B,
                                                   int32_t T);
int rglru_local_attention_block(const rglru_attn_params *a, int32_t B, int32_t T,
                                const void *x_in, void *out, void *workspace, size_t ws_bytes,
                                void *stream);

/*
 * The residual layer around a temporal-mixing block.  Operation: the page "Gemma 詳解：
 * RecurrentGemma 架構" (module printout; sections "含遞迴區塊的殘差區塊" and "含區域 MQA 的殘差
 * 區塊") wraps each block in a pre-norm residual layer with an MLP:
 *   h   = x + temporal(RMSNorm_1(x))
 *   out = h + down_proj(gelu_tanh(gate_proj(RMSNorm_2(h))) * up_proj(RMSNorm_2(h)))
 *   RMSNorm(v) = v / sqrt(mean(v^2) + eps) * scale   (per row of D_model, fp32 arithmetic)
 * scale is the per-channel multiplier itself (a model that stores w with multiplier 1 + w passes
 * 1 + w).  bf16 storage only; like a bf16 model, every step's result is rounded to bf16 (RNE):
 * the normalised rows, the block output, h, the MLP's gate, up and their product, its output.
 */
typedef struct rglru_norm_params {
    const void *temporal_scale; /* [D_model], before the temporal block */
    const void *channel_scale;  /* [D_model], before the MLP */
    float eps;
} rglru_norm_params;

/* The MLP: gate_w, up_w [F][D_model], down_w [D_model][F] ([out][in]); biases [F], [F],
 * [D_model] or NULL.  D_model % 256 == 0 and F % 256 == 0 (below 2^21), else
 * RGLRU_ERR_UNSUPPORTED. */
typedef struct rglru_mlp_params {
    int32_t D_model;
    int32_t F;
    const void *gate_w;
    const void *gate_b;
    const void *up_w;
    const void *up_b;
    const void *down_w;
    const void *down_b;
} rglru_mlp_params;

/*
 * RMSNorm with an optional residual addition, over M rows of D (bf16):
 *   h = x + residual (x alone when residual is NULL), rounded to bf16, written to h_out if given;
 *   out = RMSNorm(h) * scale, written if out is given (scale is then required).
 * M >= 0, D % 8 == 0 and D <= 8192 (else RGLRU_ERR_UNSUPPORTED), eps >= 0.  h_out and out must
 * not overlap each other or the inputs, except that h_out may be x itself (in-place add).
 */
int rglru_rmsnorm(int32_t M, int32_t D, const void *x, const void *residual, const void *scale,
                  float eps, void *h_out, void *out, void *stream);

/* The MLP alone over M rows: out [M][D_model] = down(gelu_tanh(gate(x)) * up(x)), x [M][D_model].
 * workspace: at least rglru_mlp_workspace_bytes(M, F) (gate and up outputs, [2][M][F] bf16). */
size_t rglru_mlp_workspace_bytes(int32_t M, int32_t F);
int rglru_mlp(const rglru_mlp_params *m, int32_t M, const void *x, void *out, void *workspace,
              size_t ws_bytes, void *stream);

/*
 * The residual layer around the recurrent block (prefill over T tokens): temporal is
 * rglru_block_prefill's operation (with its state arguments, as there).  x_in, out
 * [B][T][D_model].  The workspace starts with the recurrent block's own workspace; no
 * initialisation is needed.  out must not overlap x_in.
 */
size_t rglru_recurrent_layer_workspace_bytes(int32_t B, int32_t T, int32_t D, int32_t n_heads,
                                             int32_t D_model, int32_t F);
int rglru_recurrent_layer_prefill(const rglru_params *p, const rglru_proj_params *q,
                                  const rglru_norm_params *nrm, const rglru_mlp_params *m,
                                  int32_t B, int32_t T, const void *x_in, void *out,
                                  const float *h0, float *h_last, const void *conv0,
                                  void *conv_last, void *workspace, size_t ws_bytes, void *stream);

/*
 * The residual layer around the local-attention block (prefill over T tokens): temporal is
 * rglru_local_attention_block's operation; kcache, vcache (optional, as in
 * rglru_local_attention) receive the last window positions for decoding.  out must not overlap
 * x_in.  No initialisation of the workspace is needed.
 */
size_t rglru_attention_layer_workspace_bytes(const rglru_attn_params *a, int32_t B, int32_t T,
                                             int32_t F);
int rglru_attention_layer_prefill(const rglru_attn_params *a, const rglru_norm_params *nrm,
                                  const rglru_mlp_params *m, int32_t B, int32_t T,
                                  const void *x_in, void *out, void *kcache, void *vcache,
                                  void *workspace, size_t ws_bytes, void *stream);

/*
 * Decode step of the residual layer around the recurrent block: one token for each of N
 * sequences, the block's state carried in h [N][D] (fp32) and conv_state [N][3][D] (bf16) as in
 * rglru_decode_step.  x_t, out_t [N][D_model] (bf16).  The projections run as GEMMs over the N
 * rows.  workspace: at least rglru_recurrent_layer_decode_workspace_bytes(N, D, D_model, F), no
 * initialisation needed.  out_t must not overlap x_t; nothing else may overlap.
 */
size_t rglru_recurrent_layer_decode_workspace_bytes(int32_t N, int32_t D, int32_t D_model,
                                                    int32_t F);
int rglru_recurrent_layer_decode(const rglru_params *p, const rglru_proj_params *q,
                                 const rglru_norm_params *nrm, const rglru_mlp_params *m,
                                 int32_t N, const void *x_t, void *out_t, float *h,
                                 void *conv_state, void *workspace, size_t ws_bytes,
                                 void *stream);

/*
 * Decode step of the residual layer around the local-attention block: one token for each of N
 * sequences at positions pos [N] (device int32), with the ring caches of
 * rglru_local_attention_decode (n_heads <= 16).  x_t, out_t [N][D_model].  workspace: at least
 * rglru_attention_layer_decode_workspace_bytes(a, N, F), no initialisation needed.
 */
size_t rglru_attention_layer_decode_workspace_bytes(const rglru_attn_params *a, int32_t N,
                                                    int32_t F);
int rglru_attention_layer_decode(const rglru_attn_params *a, const rglru_norm_params *nrm,
                                 const rglru_mlp_params *m, int32_t N, const int32_t *pos,
                                 const void *x_t, void *out_t, void *kcache, void *vcache,
                                 void *workspace, size_t ws_bytes, void *stream);

/*
 * Backward pass of the path, for training: the gradients of
 *   L = sum_t dout_t . out_t + dh_last . h_last
 * with respect to every input of rglru_prefill (the pages give no training detail; these are the
 * chain-rule gradients of the forward operation above).
 *   x, y, dout     [B][T][D] (bf16);  h0 [B][D] fp32 or NULL;  conv0 [B][3][D] or NULL;
 *   dh_last        [B][D] fp32 or NULL (NULL = 0)
 *   dx, dy         [B][T][D] (bf16)
 *   dconv_w [D][4], dconv_b [D], dwa and dwx [H][bs][bs], dba and dbx [D], dlambda [D],
 *   dh0 [B][D], dconv0 [B][3][D]   all fp32, overwritten (not accumulated)
 *   workspace      at least rglru_prefill_backward_workspace_bytes(B, T, D, n_heads); no
 *                  initialisation needed
 * bf16 storage, block size 256, T % 32 == 0 and B * T % 256 == 0 with B * T >= 256, else
 * RGLRU_ERR_UNSUPPORTED.  Outputs must not overlap each other, the inputs or the workspace.
 * Deterministic (sums over tokens are taken in a fixed order).
 */
size_t rglru_prefill_backward_workspace_bytes(int32_t B, int32_t T, int32_t D, int32_t n_heads);
int rglru_prefill_backward(const rglru_params *p, int32_t B, int32_t T, const void *x,
                           const void *y, const float *h0, const void *conv0, const void *dout,
                           const float *dh_last, void *dx, void *dy, float *dconv_w,
                           float *dconv_b, float *dwa, float *dba, float *dwx, float *dbx,
                           float *dlambda, float *dh0, float *dconv0, void *workspace,
                           size_t ws_bytes, void *stream);

/*
 * Diagnostics of a prefill workspace: copies the error flags of the latest prefill call on it
 * to *flags_out (0 = none) and clears them.  Synchronous (waits for `stream`).  Bit 0: a carry
 * wait exceeded its bound (the affected outputs are NaN).  The next prefill call clears the
 * flags in any case.
 */
int rglru_prefill_workspace_flags(void *workspace, size_t ws_bytes, uint32_t *flags_out,
                                  void *stream);

const char *rglru_status_string(int status);
int rglru_last_hip_error(void); /* hipError_t of this thread's last failing HIP call */
int rglru_abi_version(void);    /* RGLRU_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* RGLRU_H */
