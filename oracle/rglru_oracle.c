/*
 * rglru_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential fp64 reference for the recurrent-block
 * temporal-mixing path of RecurrentGemma.  Only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark load this file.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * What it computes, per sequence b and head hd (heads are independent):
 *
 *   The pages ("Gemma 詳解：RecurrentGemma 架構", section
 *   "含遞迴區塊的殘差區塊", and the module printout on that page) fix the
 *   dataflow: two width-2560 branches; on one, a depthwise Conv1d with
 *   kernel 4 (padding 3, groups = width, with bias) followed by the
 *   RG-LRU; on the other, GELU with the tanh approximation
 *   (PytorchGELUTanh); the two branches are multiplied elementwise.
 *   The library's inputs are the two branch projections' outputs
 *   x = linear_x(.) and y = linear_y(.).
 *
 *   The pages name the RG-LRU (section "模型寬度與 RNN 寬度": it keeps a
 *   fixed-size state of RNN width) but print none of its arithmetic.  The
 *   recurrence below is the RG-LRU of the Griffin paper (arXiv 2402.19427,
 *   linked from the article "RecurrentGemma vs 传统LLM..."), restated:
 *     r_t = sigmoid(W_a u_t + b_a), i_t = sigmoid(W_x u_t + b_x)
 *     a_t = sigmoid(Lambda) ** (8 r_t)
 *     h_t = a_t h_{t-1} + sqrt(1 - a_t^2) (i_t u_t)
 *   with block-diagonal W_a, W_x (one bs x bs block per head).
 *
 * Readings where the pages are silent (each one is listed in the design doc):
 *   - the gates read the RG-LRU input u_t (the conv output);
 *   - the conv is causal: the first T of the T+3 padded outputs are kept,
 *     tap j multiplies x_{t-3+j}, and the carried conv state holds the
 *     last three conv inputs, oldest first (zeros when absent);
 *   - gate block h is stored like a Linear weight, [out j][in k]:
 *       pre[h*bs + j] = b[h*bs + j] + sum_k W[h][j][k] * u[h*bs + k];
 *   - out_t = h_t * gelu_tanh(y_t); no resets; h0 = 0 when absent.
 *
 * Everything is evaluated literally in double precision.  Inputs stored as
 * bf16 are widened exactly by placing the 16 bits in the top half of a
 * float; fp32 inputs are widened exactly.
 *
 * The dense projections around the path (same page and section, and the
 * module printout: linear_x and linear_y, width 2560 -> 2560 with bias,
 * both applied to the block input; linear_out, 2560 -> 2560 with bias,
 * applied to the product of the two branches) are plain Linear layers:
 *   out[n] = b[n] + sum_k W[n][k] in[k],   W stored [out][in].
 * oracle_block_prefill composes them with the path:
 *   out = linear_out( path( linear_x(x_in), linear_y(x_in) ) )
 * with every intermediate kept in double precision.
 *
 * The file ends with the model's other temporal-mixing block, local sliding-window
 * multi-query attention with rotary position embedding (see its section header).
 *
 * Parity pins (tests/test_oracle_pins.py): every function here is pinned
 * by closed forms, library routines or brute force; see that file.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2 /* intermediates of the composed block only */

/* Exact widening of one stored element to double. */
static double widen(const void *base, size_t idx, int dtype) {
    if (dtype == ORACLE_F64) return ((const double *)base)[idx];
    if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* GELU, tanh form (Hendrycks & Gimpel 2016): 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))). */
double oracle_gelu_tanh(double y) {
    const double k = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * y * (1.0 + tanh(k * (y + 0.044715 * y * y * y)));
}

/* Parameters of one recurrent block (all pointers are host memory). */
typedef struct {
    int dtype;        /* storage type of the conv state and all weights but Lambda */
    int xdtype;       /* type of x and y: the storage type, or ORACLE_F64 inside the block */
    int D, H, bs;     /* channels, gate heads, block size D/H */
    const void *conv_w;   /* [D][4] */
    const void *conv_b;   /* [D] or NULL */
    const void *wa, *ba;  /* [H][bs][bs] ([out][in]), [D] or NULL */
    const void *wx, *bx;
    const float *lambda;  /* [D] */
} prm_t;

/* Causal depthwise conv, one channel, one step.  win[0..2] hold the three
 * previous inputs, oldest first; tap j multiplies x_{t-3+j}. */
static double conv_step(const prm_t *p, int c, double win[3], double xt) {
    double acc = p->conv_b ? widen(p->conv_b, (size_t)c, p->dtype) : 0.0;
    acc += widen(p->conv_w, (size_t)c * 4 + 0, p->dtype) * win[0];
    acc += widen(p->conv_w, (size_t)c * 4 + 1, p->dtype) * win[1];
    acc += widen(p->conv_w, (size_t)c * 4 + 2, p->dtype) * win[2];
    acc += widen(p->conv_w, (size_t)c * 4 + 3, p->dtype) * xt;
    win[0] = win[1];
    win[1] = win[2];
    win[2] = xt;
    return acc;
}

/* Gate pre-activations of head hd for one token: u_head[bs] -> ra[bs], ri[bs]. */
static void gate_preacts(const prm_t *p, int hd, const double *u_head, double *ra, double *ri) {
    const int bs = p->bs;
    for (int j = 0; j < bs; ++j) {
        const size_t ch = (size_t)hd * bs + j;
        double sa = p->ba ? widen(p->ba, ch, p->dtype) : 0.0;
        double sx = p->bx ? widen(p->bx, ch, p->dtype) : 0.0;
        for (int k = 0; k < bs; ++k) {
            const size_t widx = ((size_t)hd * bs + j) * bs + k;
            sa += widen(p->wa, widx, p->dtype) * u_head[k];
            sx += widen(p->wx, widx, p->dtype) * u_head[k];
        }
        ra[j] = sa;
        ri[j] = sx;
    }
}

/* One RG-LRU step for one channel: returns the new state. */
static double rglru_step(double lambda, double ra, double ri, double u, double h_prev) {
    const double r = sigmoid(ra);
    const double i = sigmoid(ri);
    const double a = pow(sigmoid(lambda), 8.0 * r);
    const double m = sqrt(1.0 - a * a);
    return a * h_prev + m * (i * u);
}

/*
 * The core loop: one (sequence, head) unit over n_tok tokens.
 *   x_row(t), y_row(t): element c of token t is x[xoff + t*xstride + c].
 *   h[bs], win[3][bs]: state in/out (fp64).
 *   out[t*bs + c] receives h_t * gelu(y_t) for channel hd*bs + c.
 */
static void run_unit(const prm_t *p, int hd, int n_tok,
                     const void *x, size_t xoff, size_t xstride,
                     const void *y, size_t yoff, size_t ystride,
                     double *h, double *win, double *out) {
    const int bs = p->bs;
    double *u = (double *)malloc(sizeof(double) * 3 * (size_t)bs);
    double *ra = u + bs, *ri = u + 2 * bs;
    for (int t = 0; t < n_tok; ++t) {
        for (int c = 0; c < bs; ++c) {
            const int ch = hd * bs + c;
            double w3[3] = {win[0 * bs + c], win[1 * bs + c], win[2 * bs + c]};
            const double xt = widen(x, xoff + (size_t)t * xstride + ch, p->xdtype);
            u[c] = conv_step(p, ch, w3, xt);
            win[0 * bs + c] = w3[0];
            win[1 * bs + c] = w3[1];
            win[2 * bs + c] = w3[2];
        }
        gate_preacts(p, hd, u, ra, ri);
        for (int c = 0; c < bs; ++c) {
            const int ch = hd * bs + c;
            h[c] = rglru_step((double)p->lambda[ch], ra[c], ri[c], u[c], h[c]);
            const double yt = widen(y, yoff + (size_t)t * ystride + ch, p->xdtype);
            out[(size_t)t * bs + c] = h[c] * oracle_gelu_tanh(yt);
        }
    }
    free(u);
}

static int make_prm(prm_t *p, int dtype, int D, int H, const void *conv_w, const void *conv_b,
                    const void *wa, const void *ba, const void *wx, const void *bx,
                    const float *lambda) {
    if (D <= 0 || H <= 0 || D % H != 0) return 2;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return 3;
    if (!conv_w || !wa || !wx || !lambda) return 1;
    p->dtype = dtype;
    p->xdtype = dtype;
    p->D = D;
    p->H = H;
    p->bs = D / H;
    p->conv_w = conv_w;
    p->conv_b = conv_b;
    p->wa = wa;
    p->ba = ba;
    p->wx = wx;
    p->bx = bx;
    p->lambda = lambda;
    return 0;
}

/* Initial state of unit (b, hd): h from h0 (fp32) or zero, window from conv0 or zero. */
static void init_state(const prm_t *p, int b, int hd, const float *h0, const void *conv0,
                       double *h, double *win) {
    const int bs = p->bs, D = p->D;
    for (int c = 0; c < bs; ++c) {
        const size_t ch = (size_t)hd * bs + c;
        h[c] = h0 ? (double)h0[(size_t)b * D + ch] : 0.0;
        for (int j = 0; j < 3; ++j)
            win[j * bs + c] = conv0 ? widen(conv0, ((size_t)b * 3 + j) * D + ch, p->dtype) : 0.0;
    }
}

/*
 * Prefill of one (b, hd) unit over the first T_use tokens of x, y [B][T][D].
 * out_unit [T_use][bs]; h_end [bs]; conv_end [3][bs] (state after T_use tokens).
 */
int oracle_prefill_unit(int dtype, int T, int D, int H, int b, int hd, int T_use,
                        const void *x, const void *y, const void *conv_w, const void *conv_b,
                        const void *wa, const void *ba, const void *wx, const void *bx,
                        const float *lambda, const float *h0, const void *conv0,
                        double *out_unit, double *h_end, double *conv_end) {
    prm_t p;
    int st = make_prm(&p, dtype, D, H, conv_w, conv_b, wa, ba, wx, bx, lambda);
    if (st) return st;
    if (T < 0 || T_use < 0 || T_use > T || hd < 0 || hd >= H || b < 0) return 2;
    init_state(&p, b, hd, h0, conv0, h_end, conv_end);
    run_unit(&p, hd, T_use, x, (size_t)b * T * D, (size_t)D, y, (size_t)b * T * D, (size_t)D,
             h_end, conv_end, out_unit);
    return 0;
}

/*
 * Full prefill: x, y [B][T][D]; out [B][T][D], h_last [B][D], conv_last [B][3][D]
 * (all outputs fp64).  Units (b, hd) run in parallel over nthreads threads.
 */
static void prefill_all(const prm_t *pp, int B, int T, const void *x, const void *y,
                        const float *h0, const void *conv0, double *out, double *h_last,
                        double *conv_last, int nthreads) {
    const prm_t p = *pp;
    const int D = p.D, H = p.H;
    const int bs = p.bs;
    const int n_units = B * H;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int unit = 0; unit < n_units; ++unit) {
        const int b = unit / H, hd = unit % H;
        double *h = (double *)malloc(sizeof(double) * 4 * (size_t)bs);
        double *win = h + bs;
        double *o = (double *)malloc(sizeof(double) * ((size_t)T * bs + 1));
        init_state(&p, b, hd, h0, conv0, h, win);
        run_unit(&p, hd, T, x, (size_t)b * T * D, (size_t)D, y, (size_t)b * T * D, (size_t)D, h,
                 win, o);
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < bs; ++c)
                out[((size_t)b * T + t) * D + (size_t)hd * bs + c] = o[(size_t)t * bs + c];
        for (int c = 0; c < bs; ++c) {
            h_last[(size_t)b * D + (size_t)hd * bs + c] = h[c];
            for (int j = 0; j < 3; ++j)
                conv_last[((size_t)b * 3 + j) * D + (size_t)hd * bs + c] = win[j * bs + c];
        }
        free(o);
        free(h);
    }
}

int oracle_prefill(int dtype, int B, int T, int D, int H, const void *x, const void *y,
                   const void *conv_w, const void *conv_b, const void *wa, const void *ba,
                   const void *wx, const void *bx, const float *lambda, const float *h0,
                   const void *conv0, double *out, double *h_last, double *conv_last,
                   int nthreads) {
    prm_t p;
    int st = make_prm(&p, dtype, D, H, conv_w, conv_b, wa, ba, wx, bx, lambda);
    if (st) return st;
    if (B < 1 || T < 0) return 2;
    prefill_all(&p, B, T, x, y, h0, conv0, out, h_last, conv_last, nthreads);
    return 0;
}

/*
 * A Linear layer over M rows: in [M][K] (type xdtype), W [N][K] ([out][in], storage type
 * wdtype), b [N] or NULL; out [M][N] = b + in W^T, summed in k order in double precision.
 */
static void linear_rows(int M, int K, int N, const void *in, int xdtype, const void *w,
                        const void *b, int wdtype, double *out) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int m = 0; m < M; ++m) {
        for (int n = 0; n < N; ++n) {
            double s = b ? widen(b, (size_t)n, wdtype) : 0.0;
            for (int k = 0; k < K; ++k)
                s += widen(w, (size_t)n * K + k, wdtype) * widen(in, (size_t)m * K + k, xdtype);
            out[(size_t)m * N + n] = s;
        }
    }
}

/* One Linear layer: x [M][K] (storage dtype), W [N][K], b [N] or NULL -> out [M][N] fp64. */
int oracle_linear(int dtype, int M, int K, int N, const void *x, const void *w, const void *b,
                  double *out) {
    if (M < 0 || K < 1 || N < 1) return 2;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return 3;
    if (!x || !w || !out) return 1;
    linear_rows(M, K, N, x, dtype, w, b, dtype, out);
    return 0;
}

/*
 * The whole recurrent block's temporal mixing over T tokens:
 *   x_in [B][T][Dm] (type xdtype: the storage type, or fp64 inside a residual layer)
 *   -> xb = linear_x(x_in), yb = linear_y(x_in)                             [B][T][D] fp64
 *   -> the path above (conv, RG-LRU, times GELU of yb)                      [B][T][D] fp64
 *   -> out = linear_out(.)                                                  [B][T][Dm] fp64
 * lx_w, ly_w [D][Dm]; lo_w [Dm][D]; biases [D], [D], [Dm] or NULL.  h_last [B][D] and
 * conv_last [B][3][D] (fp64) are the path's final state; conv0 holds storage-type values.
 */
int oracle_block_prefill(int dtype, int xdtype, int B, int T, int Dm, int D, int H,
                         const void *x_in,
                         const void *lx_w, const void *lx_b, const void *ly_w, const void *ly_b,
                         const void *lo_w, const void *lo_b, const void *conv_w,
                         const void *conv_b, const void *wa, const void *ba, const void *wx,
                         const void *bx, const float *lambda, const float *h0,
                         const void *conv0, double *out, double *h_last, double *conv_last,
                         int nthreads) {
    prm_t p;
    int st = make_prm(&p, dtype, D, H, conv_w, conv_b, wa, ba, wx, bx, lambda);
    if (st) return st;
    if (B < 1 || T < 0 || Dm < 1) return 2;
    if (xdtype != dtype && xdtype != ORACLE_F64) return 3;
    if (!x_in || !lx_w || !ly_w || !lo_w) return 1;
    const size_t MD = (size_t)B * T * D;
    double *xb = (double *)malloc(sizeof(double) * (3 * MD + 1));
    if (!xb) return 1;
    double *yb = xb + MD, *mg = yb + MD;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    linear_rows(B * T, Dm, D, x_in, xdtype, lx_w, lx_b, dtype, xb);
    linear_rows(B * T, Dm, D, x_in, xdtype, ly_w, ly_b, dtype, yb);
    p.xdtype = ORACLE_F64;
    prefill_all(&p, B, T, xb, yb, h0, conv0, mg, h_last, conv_last, nthreads);
    linear_rows(B * T, D, Dm, mg, ORACLE_F64, lo_w, lo_b, dtype, out);
    free(xb);
    return 0;
}

/*
 * One decode step for N sequences: x_t, y_t [N][D] (storage dtype);
 * h [N][D] and win [N][3][D] are fp64 state, updated in place; out_t [N][D].
 * The body is the prefill loop with one token.
 */
int oracle_decode_step(int dtype, int N, int D, int H, const void *x_t, const void *y_t,
                       const void *conv_w, const void *conv_b, const void *wa, const void *ba,
                       const void *wx, const void *bx, const float *lambda, double *h,
                       double *win, double *out_t) {
    prm_t p;
    int st = make_prm(&p, dtype, D, H, conv_w, conv_b, wa, ba, wx, bx, lambda);
    if (st) return st;
    if (N < 1) return 2;
    const int bs = p.bs;
    double *hu = (double *)malloc(sizeof(double) * 5 * (size_t)bs);
    double *wu = hu + bs, *ou = hu + 4 * bs;
    for (int n = 0; n < N; ++n) {
        for (int hd = 0; hd < H; ++hd) {
            for (int c = 0; c < bs; ++c) {
                const size_t ch = (size_t)hd * bs + c;
                hu[c] = h[(size_t)n * D + ch];
                for (int j = 0; j < 3; ++j) wu[j * bs + c] = win[((size_t)n * 3 + j) * D + ch];
            }
            run_unit(&p, hd, 1, x_t, (size_t)n * D, 0, y_t, (size_t)n * D, 0, hu, wu, ou);
            for (int c = 0; c < bs; ++c) {
                const size_t ch = (size_t)hd * bs + c;
                h[(size_t)n * D + ch] = hu[c];
                for (int j = 0; j < 3; ++j) win[((size_t)n * 3 + j) * D + ch] = wu[j * bs + c];
                out_t[(size_t)n * D + ch] = ou[c];
            }
        }
    }
    free(hu);
    return 0;
}

/*
 * Conv-state update: x_new [N][T_new][D] (storage dtype); win [N][3][D] fp64
 * state updated in place to the last three inputs; conv_out [N][T_new][D]
 * (fp64) receives the conv outputs (may be NULL).
 */
int oracle_conv1d_state_update(int dtype, int N, int T_new, int D, const void *x_new,
                               const void *conv_w, const void *conv_b, double *win,
                               double *conv_out) {
    prm_t p;
    memset(&p, 0, sizeof p);
    if (N < 1 || T_new < 0 || D < 1) return 2;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return 3;
    if (!conv_w || !x_new || !win) return 1;
    p.dtype = dtype;
    p.xdtype = dtype;
    p.D = D;
    p.conv_w = conv_w;
    p.conv_b = conv_b;
    for (int n = 0; n < N; ++n) {
        for (int c = 0; c < D; ++c) {
            double w3[3];
            for (int j = 0; j < 3; ++j) w3[j] = win[((size_t)n * 3 + j) * D + c];
            for (int t = 0; t < T_new; ++t) {
                const double xt = widen(x_new, ((size_t)n * T_new + t) * D + c, dtype);
                const double u = conv_step(&p, c, w3, xt);
                if (conv_out) conv_out[((size_t)n * T_new + t) * D + c] = u;
            }
            for (int j = 0; j < 3; ++j) win[((size_t)n * 3 + j) * D + c] = w3[j];
        }
    }
    return 0;
}

/* Gate pre-activations for n_tok tokens: u [n_tok][D] (fp64) -> ra, ri [n_tok][D]. */
int oracle_gate_preacts(int dtype, int n_tok, int D, int H, const double *u, const void *wa,
                        const void *ba, const void *wx, const void *bx, double *ra, double *ri) {
    prm_t p;
    static const float dummy_lambda = 0.0f;
    static const float dummy_w = 0.0f;
    int st = make_prm(&p, dtype, D, H, &dummy_w, NULL, wa, ba, wx, bx, &dummy_lambda);
    if (st) return st;
    for (int t = 0; t < n_tok; ++t)
        for (int hd = 0; hd < H; ++hd)
            gate_preacts(&p, hd, u + (size_t)t * D + (size_t)hd * p.bs,
                         ra + (size_t)t * D + (size_t)hd * p.bs,
                         ri + (size_t)t * D + (size_t)hd * p.bs);
    return 0;
}

/* One RG-LRU step on plain doubles (exposed so the pins can probe it directly). */
double oracle_rglru_step(double lambda, double ra, double ri, double u, double h_prev) {
    return rglru_step(lambda, ra, ri, u, h_prev);
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ======================================================================================
 * Local sliding-window multi-query attention: the other temporal-mixing block of the same
 * model (page "Gemma 詳解：RecurrentGemma 架構", section "含區域 MQA 的殘差區塊" and the
 * printout's RecurrentGemmaSdpaAttention): q_proj (width -> Hq heads of dh, no bias),
 * k_proj and v_proj (width -> one head of dh shared by all query heads, no bias), rotary
 * position embedding on q and k following the base Gemma model, each position attending to a
 * fixed window of past tokens (section "區域注意力視窗大小": 2k tokens), and o_proj (with bias).
 *
 * Readings (listed in the design doc):
 *   - RoPE pairs dimension i with i + dh/2 (the rotate-half convention) and turns pair i by
 *     pos * base^(-2 i / dh), base 10000, over the whole head; pos is the token's index in
 *     its sequence, from 0;
 *   - the window of W tokens is the current token and the W - 1 before it;
 *   - scores are q.k / sqrt(dh), no soft-capping; softmax over the window.
 * ====================================================================================== */

/* RoPE of one head vector v[dh] at position pos, in place. */
static void rope_head(double *v, int dh, double pos, double base) {
    const int half = dh / 2;
    for (int i = 0; i < half; ++i) {
        const double theta = pos * pow(base, -2.0 * (double)i / (double)dh);
        const double c = cos(theta), s = sin(theta);
        const double a = v[i], b = v[i + half];
        v[i] = a * c - b * s;
        v[i + half] = b * c + a * s;
    }
}

/* RoPE of n head vectors v[n][dh] at positions pos[n], in place. */
int oracle_rope(int n, int dh, const double *pos, double base, double *v) {
    if (n < 0 || dh < 2 || dh % 2 != 0) return 2;
    for (int r = 0; r < n; ++r) rope_head(v + (size_t)r * dh, dh, pos[r], base);
    return 0;
}

/* Attention of one query vector q[dh] over keys/values k, v [n][dh] (all in the window):
 * o[dh] = sum_s softmax_s(q . k_s / sqrt(dh)) v_s. */
static void attend_one(int n, int dh, const double *q, const double *k, const double *v,
                       double *o, double *score) {
    const double scale = 1.0 / sqrt((double)dh);
    double mx = -INFINITY;
    for (int s = 0; s < n; ++s) {
        double d = 0.0;
        for (int c = 0; c < dh; ++c) d += q[c] * k[(size_t)s * dh + c];
        score[s] = d * scale;
        if (score[s] > mx) mx = score[s];
    }
    double den = 0.0;
    for (int s = 0; s < n; ++s) {
        score[s] = exp(score[s] - mx);
        den += score[s];
    }
    for (int c = 0; c < dh; ++c) o[c] = 0.0;
    for (int s = 0; s < n; ++s)
        for (int c = 0; c < dh; ++c) o[c] += (score[s] / den) * v[(size_t)s * dh + c];
}

/* Local MQA over one sequence of T tokens: q [T][Hq][dh], k, v [T][dh] (positions already
 * encoded); o [T][Hq][dh].  Query t of every head attends to tokens max(0, t-W+1) .. t. */
int oracle_local_mqa(int T, int Hq, int dh, int W, const double *q, const double *k,
                     const double *v, double *o) {
    if (T < 0 || Hq < 1 || dh < 1 || W < 1) return 2;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int t = 0; t < T; ++t) {
        double *score = (double *)malloc(sizeof(double) * ((size_t)W + 1));
        const int s0 = t - W + 1 > 0 ? t - W + 1 : 0;
        for (int h = 0; h < Hq; ++h)
            attend_one(t - s0 + 1, dh, q + ((size_t)t * Hq + h) * dh, k + (size_t)s0 * dh,
                       v + (size_t)s0 * dh, o + ((size_t)t * Hq + h) * dh, score);
        free(score);
    }
    return 0;
}

/*
 * The local-attention temporal-mixing block over B sequences of T tokens:
 *   x_in [B][T][Dm] (type xdtype: storage, or fp64 inside a residual layer) -> q = x Wq^T [.., Hq*dh], k = x Wk^T [.., dh], v = x Wv^T
 *   (no biases) -> RoPE on q (each head) and k at positions 0 .. T-1 -> local MQA with window
 *   W -> out = o Wo^T + bo  [B][T][Dm] (fp64).  Wq [Hq*dh][Dm], Wk, Wv [dh][Dm], Wo [Dm][Hq*dh].
 */
int oracle_local_attention_block(int dtype, int xdtype, int B, int T, int Dm, int Hq, int dh,
                                 int W, double base, const void *x_in, const void *wq,
                                 const void *wk, const void *wv, const void *wo, const void *bo,
                                 double *out, int nthreads) {
    if (B < 1 || T < 0 || Dm < 1 || Hq < 1 || dh < 2 || dh % 2 || W < 1) return 2;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return 3;
    if (xdtype != dtype && xdtype != ORACLE_F64) return 3;
    if (!x_in || !wq || !wk || !wv || !wo || !out) return 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    const int DQ = Hq * dh;
    const size_t M = (size_t)T;
    double *q = (double *)malloc(sizeof(double) * (M * DQ + 1));
    double *k = (double *)malloc(sizeof(double) * (M * dh + 1));
    double *v = (double *)malloc(sizeof(double) * (M * dh + 1));
    double *o = (double *)malloc(sizeof(double) * (M * DQ + 1));
    if (!q || !k || !v || !o) return 1;
    for (int b = 0; b < B; ++b) {
        const size_t xoff = (size_t)b * T * Dm;
        const size_t xes = xdtype == ORACLE_F64 ? 8 : (xdtype == ORACLE_F32 ? 4 : 2);
        const void *xb = (const char *)x_in + xoff * xes;
        linear_rows(T, Dm, DQ, xb, xdtype, wq, NULL, dtype, q);
        linear_rows(T, Dm, dh, xb, xdtype, wk, NULL, dtype, k);
        linear_rows(T, Dm, dh, xb, xdtype, wv, NULL, dtype, v);
        for (int t = 0; t < T; ++t) {
            for (int h = 0; h < Hq; ++h) rope_head(q + ((size_t)t * Hq + h) * dh, dh, (double)t, base);
            rope_head(k + (size_t)t * dh, dh, (double)t, base);
        }
        oracle_local_mqa(T, Hq, dh, W, q, k, v, o);
        linear_rows(T, DQ, Dm, o, ORACLE_F64, wo, bo, dtype, out + xoff);
    }
    free(q);
    free(k);
    free(v);
    free(o);
    return 0;
}

/* ======================================================================================
 * The residual layer's other parts: the page "Gemma 詳解：RecurrentGemma 架構" (module
 * printout; sections "含遞迴區塊的殘差區塊" and "含區域 MQA 的殘差區塊") puts an RMSNorm
 * (temporal_pre_norm) before the temporal-mixing block and another (channel_pre_norm) before
 * the MLP, whose gate_proj and up_proj (width -> 3 x width, with bias), GELU-tanh act_fn and
 * down_proj (back to the width, with bias) follow the base Gemma feed-forward layer.
 *
 * Readings (listed in the design doc):
 *   - RMSNorm(x) = x / sqrt(mean_d x_d^2 + eps) * g, with g the per-channel scale (models that
 *     store w with g = 1 + w pass 1 + w); eps is an argument (1e-6 in the tests);
 *   - MLP(x) = down_proj(gelu_tanh(gate_proj(x)) * up_proj(x)): the activation is applied to
 *     the gate branch only;
 *   - the layer is pre-norm with two residual additions:
 *       h = x + temporal(RMSNorm_1(x)),  out = h + MLP(RMSNorm_2(h)).
 * ====================================================================================== */

/* RMSNorm over rows of D: x [rows][D] (type xdtype), g [D] (type wdtype) -> out fp64. */
int oracle_rmsnorm(int xdtype, int wdtype, int rows, int D, const void *x, const void *g,
                   double eps, double *out) {
    if (rows < 0 || D < 1 || !(eps >= 0.0)) return 2;
    if (!x || !g || !out) return 1;
    for (int r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int d = 0; d < D; ++d) {
            const double v = widen(x, (size_t)r * D + d, xdtype);
            ss += v * v;
        }
        const double inv = 1.0 / sqrt(ss / (double)D + eps);
        for (int d = 0; d < D; ++d)
            out[(size_t)r * D + d] = widen(x, (size_t)r * D + d, xdtype) * inv * widen(g, d, wdtype);
    }
    return 0;
}

/* The gated MLP over rows: x [rows][Dm] (type xdtype); gate_w, up_w [F][Dm], down_w [Dm][F]
 * ([out][in], type wdtype); biases [F], [F], [Dm] or NULL -> out [rows][Dm] fp64. */
int oracle_mlp(int xdtype, int wdtype, int rows, int Dm, int F, const void *x, const void *gw,
               const void *gb, const void *uw, const void *ub, const void *dw, const void *db,
               double *out, int nthreads) {
    if (rows < 0 || Dm < 1 || F < 1) return 2;
    if (!x || !gw || !uw || !dw || !out) return 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    const size_t n = (size_t)rows * F;
    double *gt = (double *)malloc(sizeof(double) * (2 * n + 1));
    if (!gt) return 1;
    double *up = gt + n;
    linear_rows(rows, Dm, F, x, xdtype, gw, gb, wdtype, gt);
    linear_rows(rows, Dm, F, x, xdtype, uw, ub, wdtype, up);
    for (size_t i = 0; i < n; ++i) gt[i] = oracle_gelu_tanh(gt[i]) * up[i];
    linear_rows(rows, F, Dm, gt, ORACLE_F64, dw, db, wdtype, out);
    free(gt);
    return 0;
}

/* ======================================================================================
 * Backward pass of the path (for training).  The pages give no training detail; the
 * gradients are those of the forward definition above, by the chain rule, for the loss
 *   L = sum_t dout_t . out_t + dh_last . h_T-1
 * (dh_last may be absent).  Per (sequence, head) the forward is re-run keeping u, r, i, a, m
 * and h for every token; then time runs backwards:
 *   dh_t   = dh_{t+1} a_{t+1} + dout_t gelu(y_t)            (carry of the state gradient)
 *   dy_t   = dout_t h_t gelu'(y_t)
 *   v_t    = m_t i_t u_t:   du += dh m i,  dm = dh i u,  di = dh m u
 *   a_t    = sigma(L)^(8 r):  da = dh h_{t-1} - dm a / m,  dr = da a 8 log sigma(L),
 *            dL += da a 8 r (1 - sigma(L))
 *   r = sigma(W_a u + b_a), i = sigma(W_x u + b_x): dRpre = dr r (1 - r), dIpre = di i (1 - i),
 *            du += W_a^T dRpre + W_x^T dIpre, dW += dRpre u^T, db += dRpre
 *   u_t = conv_b + sum_j w_j x~_{t-3+j}:  dconv_b += du, dw_j += du x~_{t-3+j},
 *            dx~_{t-3+j} += du w_j (the three positions before 0 are the conv0 window)
 *   dh0 = the state gradient carried past t = 0.
 * All outputs are fp64 and fully written (accumulated from zero).
 * ====================================================================================== */
static double gelu_tanh_grad(double y) {
    const double k = sqrt(2.0 / 3.14159265358979323846);
    const double z = k * (y + 0.044715 * y * y * y);
    const double th = tanh(z);
    return 0.5 * (1.0 + th) + 0.5 * y * (1.0 - th * th) * k * (1.0 + 3.0 * 0.044715 * y * y);
}

int oracle_prefill_backward(int dtype, int B, int T, int D, int H, const void *x, const void *y,
                            const void *conv_w, const void *conv_b, const void *wa,
                            const void *ba, const void *wx, const void *bx, const float *lambda,
                            const float *h0, const void *conv0, const double *dout,
                            const double *dh_last, double *dx, double *dy, double *dconv_w,
                            double *dconv_b, double *dwa, double *dba, double *dwx, double *dbx,
                            double *dlambda, double *dh0, double *dconv0) {
    prm_t p;
    int st = make_prm(&p, dtype, D, H, conv_w, conv_b, wa, ba, wx, bx, lambda);
    if (st) return st;
    if (B < 1 || T < 0) return 2;
    if (!dout || !dx || !dy || !dconv_w || !dconv_b || !dwa || !dba || !dwx || !dbx ||
        !dlambda || !dh0 || !dconv0)
        return 1;
    if (T > 0 && (!x || !y)) return 1;
    const int bs = p.bs;
    const size_t BTD = (size_t)B * T * D;
    memset(dx, 0, sizeof(double) * BTD);
    memset(dy, 0, sizeof(double) * BTD);
    memset(dconv_w, 0, sizeof(double) * (size_t)D * 4);
    memset(dconv_b, 0, sizeof(double) * (size_t)D);
    memset(dwa, 0, sizeof(double) * (size_t)H * bs * bs);
    memset(dwx, 0, sizeof(double) * (size_t)H * bs * bs);
    memset(dba, 0, sizeof(double) * (size_t)D);
    memset(dbx, 0, sizeof(double) * (size_t)D);
    memset(dlambda, 0, sizeof(double) * (size_t)D);
    memset(dconv0, 0, sizeof(double) * (size_t)B * 3 * D);
    /* per-token values of one unit: window (3 per token), u, r, i, a, m, h, the two gate
     * pre-activations; then the state gradient and three per-channel scratch rows */
    const size_t per = (size_t)(T + 1) * bs;
    double *xw = (double *)malloc(sizeof(double) * (11 * per + 4 * (size_t)bs + 1));
    if (!xw) return 1;
    double *u = xw + 3 * per, *r = u + per, *ig = r + per, *a = ig + per, *m = a + per;
    double *h = m + per;            /* h[(t + 1) * bs + c], h[c] = h0 */
    double *ra = h + per, *ri = ra + per;
    double *dh = ri + per, *dra = dh + bs, *dia = dra + bs, *duv = dia + bs;
    for (int b = 0; b < B; ++b) {
        for (int hd = 0; hd < H; ++hd) {
            double win[3 * 256];
            if (bs > 256) {
                free(xw);
                return 3;
            }
            init_state(&p, b, hd, h0, conv0, h, win);   /* h[0..bs), win[j * bs + c] */
            for (int t = 0; t < T; ++t) {
                for (int c = 0; c < bs; ++c) {
                    const size_t ch = (size_t)hd * bs + c;
                    const double xt = widen(x, ((size_t)b * T + t) * D + ch, p.xdtype);
                    double w3[3] = {win[c], win[bs + c], win[2 * bs + c]};
                    xw[((size_t)t * bs + c) * 3 + 0] = w3[0];
                    xw[((size_t)t * bs + c) * 3 + 1] = w3[1];
                    xw[((size_t)t * bs + c) * 3 + 2] = w3[2];
                    u[(size_t)t * bs + c] = conv_step(&p, (int)ch, w3, xt);
                    win[c] = w3[0];
                    win[bs + c] = w3[1];
                    win[2 * bs + c] = w3[2];
                }
                gate_preacts(&p, hd, u + (size_t)t * bs, ra + (size_t)t * bs, ri + (size_t)t * bs);
                for (int c = 0; c < bs; ++c) {
                    const size_t k = (size_t)t * bs + c, ch = (size_t)hd * bs + c;
                    r[k] = sigmoid(ra[k]);
                    ig[k] = sigmoid(ri[k]);
                    a[k] = pow(sigmoid((double)lambda[ch]), 8.0 * r[k]);
                    m[k] = sqrt(1.0 - a[k] * a[k]);
                    h[k + bs] = a[k] * h[k] + m[k] * (ig[k] * u[k]);
                }
            }
            for (int c = 0; c < bs; ++c)
                dh[c] = dh_last ? dh_last[(size_t)b * D + (size_t)hd * bs + c] : 0.0;
            for (int t = T - 1; t >= 0; --t) {
                for (int c = 0; c < bs; ++c) {
                    const size_t k = (size_t)t * bs + c, ch = (size_t)hd * bs + c;
                    const size_t o = ((size_t)b * T + t) * D + ch;
                    const double yt = widen(y, o, p.xdtype);
                    const double g = dh[c] + dout[o] * oracle_gelu_tanh(yt);
                    dy[o] = dout[o] * h[k + bs] * gelu_tanh_grad(yt);
                    duv[c] = g * m[k] * ig[k];
                    const double dm = g * ig[k] * u[k];
                    const double di = g * m[k] * u[k];
                    const double da = g * h[k] - dm * a[k] / m[k];
                    const double sg = sigmoid((double)lambda[ch]);
                    dlambda[ch] += da * a[k] * 8.0 * r[k] * (1.0 - sg);
                    const double dr = da * a[k] * 8.0 * log(sg);
                    dra[c] = dr * r[k] * (1.0 - r[k]);
                    dia[c] = di * ig[k] * (1.0 - ig[k]);
                    dh[c] = g * a[k];
                }
                for (int j = 0; j < bs; ++j) {
                    const size_t ch = (size_t)hd * bs + j;
                    dba[ch] += dra[j];
                    dbx[ch] += dia[j];
                    for (int kk = 0; kk < bs; ++kk) {
                        const size_t widx = ((size_t)hd * bs + j) * bs + kk;
                        dwa[widx] += dra[j] * u[(size_t)t * bs + kk];
                        dwx[widx] += dia[j] * u[(size_t)t * bs + kk];
                        duv[kk] += widen(p.wa, widx, p.dtype) * dra[j] +
                                   widen(p.wx, widx, p.dtype) * dia[j];
                    }
                }
                for (int c = 0; c < bs; ++c) {
                    const size_t ch = (size_t)hd * bs + c;
                    const double du = duv[c];
                    dconv_b[ch] += du;
                    for (int j = 0; j < 4; ++j) {
                        const double xv = j < 3 ? xw[((size_t)t * bs + c) * 3 + j]
                                                : widen(x, ((size_t)b * T + t) * D + ch, p.xdtype);
                        dconv_w[ch * 4 + j] += du * xv;
                        const double gx = du * widen(p.conv_w, ch * 4 + j, p.dtype);
                        const int pos = t - 3 + j;
                        if (pos >= 0) dx[((size_t)b * T + pos) * D + ch] += gx;
                        else dconv0[((size_t)b * 3 + (pos + 3)) * D + ch] += gx;
                    }
                }
            }
            for (int c = 0; c < bs; ++c) dh0[(size_t)b * D + (size_t)hd * bs + c] = dh[c];
        }
    }
    free(xw);
    return 0;
}
