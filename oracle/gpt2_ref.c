/*
 * gpt2_ref.c -- the oracle: a plain, slow, obviously-correct CPU implementation
 * of one GPT-2 training step (forward, backward, AdamW), in double precision.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * headers, tables or helpers with the GPU library; the two agree only through
 * the definitions below and the seeded inputs both are given.
 *
 * What it computes follows the pages this project is built from:
 *  - "OpenAI創始大神手搓千行C代碼訓練GPT，附PyTorch遷移教程" (QbitAI), section
 *    "手動實現每個層前向/反向傳播": every layer has a hand-written forward and
 *    backward pass, chained into one loop; one flat 1-D allocation holds all
 *    weights and activations, made once at the start.
 *  - "“真男人就應該用 C 編程”！用 1000 行 C 代碼手搓了一個大模型…" (InfoQ), the
 *    layer-list paragraph (encoder, layernorm, matmul, self-attention, gelu,
 *    residual, softmax, cross-entropy) and the M3 Max run log (Adam at
 *    lr 1e-4; the printed model header and num_parameters / num_activations).
 *  - "Bản sao ChatGPT dựa trên GPT-2 được triển khai bằng 3000 byte C (2023)"
 *    (GeekNews), sections "Triển khai các lớp mạng nơ-ron" (layers: GELU,
 *    causal lower triangle, LayerNorm over mean and variance, Linear = matmul
 *    then bias on every row) and "Phần lõi Transformer" (block dataflow; final
 *    LayerNorm then a product with the token-embedding weights), and the
 *    comment thread (the tanh form of GELU with its two constants).
 *
 * Readings where the pages are silent (each listed in the design notes):
 * LayerNorm eps 1e-5 and biased variance; attention scale 1/sqrt(head dim);
 * mask u <= t (diagonal kept); GELU k = sqrt(2/pi) at full precision, 0.044715;
 * weights stored out x in, row-major; q|k|v as consecutive C-column blocks with
 * heads contiguous inside each block; tied head without bias over v < V only;
 * mean loss over all B*T positions; backward accumulates into grads; AdamW
 * (decoupled weight decay, bias correction, eps added to sqrt(v_hat), t from 1).
 *
 * Precision: every value and every accumulator is a C double.  Sums run in
 * the order the definition is written (index 0 upward).  OpenMP, when
 * enabled, splits only independent outputs across threads, so the result does
 * not depend on the thread count.
 *
 * Pins (what this file is checked against, outside itself): finite-difference
 * gradients on tiny models (the gradient-checking idea of
 * "femtoGPT: 纯Rust实现的极简生成式预训练Transformer", section "梯度检查");
 * the printed num_parameters 124439808 and num_activations 73323776; loss
 * = ln V for all-zero logits; softmax rows summing to one; LayerNorm output
 * statistics; attention and GELU closed forms; AdamW's first-step closed form;
 * and library routines (torch float64 layer_norm / gelu / attention /
 * cross_entropy) for the forward definitions; the decoding step against
 * this file's own full forward (the logits of a decoded position equal the
 * forward's at that position) and its sampler against a cumulative-sum search.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef long long i64;

/* ------------------------------------------------------------------------ */
/* parameter layout: 16 tensors, in this order, each stacked over layers     */
/* ------------------------------------------------------------------------ */

enum { REF_NUM_PARAM_TENSORS = 16 };

static const char *ref_param_names[REF_NUM_PARAM_TENSORS] = {
    "wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
    "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb"};

typedef struct {
    int maxT, V, Vp, L, NH, C;
} ref_shape;

static void param_counts(const ref_shape *s, i64 n[REF_NUM_PARAM_TENSORS]) {
    i64 C = s->C, L = s->L;
    n[0] = (i64)s->Vp * C;   /* wte: token embedding, also the tied head  */
    n[1] = (i64)s->maxT * C; /* wpe: position embedding                    */
    n[2] = L * C;            /* ln1w                                       */
    n[3] = L * C;            /* ln1b                                       */
    n[4] = L * 3 * C * C;    /* qkvw [L][3C][C]                            */
    n[5] = L * 3 * C;        /* qkvb                                       */
    n[6] = L * C * C;        /* attprojw [L][C][C]                         */
    n[7] = L * C;            /* attprojb                                   */
    n[8] = L * C;            /* ln2w                                       */
    n[9] = L * C;            /* ln2b                                       */
    n[10] = L * 4 * C * C;   /* fcw [L][4C][C]                             */
    n[11] = L * 4 * C;       /* fcb                                        */
    n[12] = L * C * 4 * C;   /* fcprojw [L][C][4C]                         */
    n[13] = L * C;           /* fcprojb                                    */
    n[14] = C;               /* lnfw                                       */
    n[15] = C;               /* lnfb                                       */
}

/* Offset and size of parameter tensor idx; returns the total count. */
i64 ref_param_tensor(int maxT, int V, int Vp, int L, int NH, int C, int idx,
                     i64 *offset, i64 *count, const char **name) {
    ref_shape s = {maxT, V, Vp, L, NH, C};
    i64 n[REF_NUM_PARAM_TENSORS];
    param_counts(&s, n);
    i64 off = 0, total = 0;
    for (int i = 0; i < REF_NUM_PARAM_TENSORS; i++) {
        if (i == idx) {
            if (offset) *offset = off;
            if (count) *count = n[i];
            if (name) *name = ref_param_names[i];
        }
        off += n[i];
    }
    total = off;
    return total;
}

int ref_num_param_tensors(void) { return REF_NUM_PARAM_TENSORS; }

/* ------------------------------------------------------------------------ */
/* saved activations: the 23-tensor set the oracle allocates                 */
/* ------------------------------------------------------------------------ */

enum {
    A_ENCODED, A_LN1, A_LN1_MEAN, A_LN1_RSTD, A_QKV, A_ATTY, A_PREATT, A_ATT,
    A_ATTPROJ, A_RESIDUAL2, A_LN2, A_LN2_MEAN, A_LN2_RSTD, A_FCH, A_FCH_GELU,
    A_FCPROJ, A_RESIDUAL3, A_LNF, A_LNF_MEAN, A_LNF_RSTD, A_LOGITS, A_PROBS,
    A_LOSSES, NUM_ACTS
};

static const char *ref_act_names[NUM_ACTS] = {
    "encoded", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "preatt", "att",
    "attproj", "residual2", "ln2", "ln2_mean", "ln2_rstd", "fch", "fch_gelu",
    "fcproj", "residual3", "lnf", "lnf_mean", "lnf_rstd", "logits", "probs",
    "losses"};

static void act_counts(const ref_shape *s, int B, int T, i64 n[NUM_ACTS]) {
    i64 L = s->L, C = s->C, NH = s->NH, BT = (i64)B * T;
    n[A_ENCODED] = BT * C;
    n[A_LN1] = L * BT * C;
    n[A_LN1_MEAN] = L * BT;
    n[A_LN1_RSTD] = L * BT;
    n[A_QKV] = L * BT * 3 * C;
    n[A_ATTY] = L * BT * C;
    n[A_PREATT] = L * B * NH * (i64)T * T;
    n[A_ATT] = L * B * NH * (i64)T * T;
    n[A_ATTPROJ] = L * BT * C;
    n[A_RESIDUAL2] = L * BT * C;
    n[A_LN2] = L * BT * C;
    n[A_LN2_MEAN] = L * BT;
    n[A_LN2_RSTD] = L * BT;
    n[A_FCH] = L * BT * 4 * C;
    n[A_FCH_GELU] = L * BT * 4 * C;
    n[A_FCPROJ] = L * BT * C;
    n[A_RESIDUAL3] = L * BT * C;
    n[A_LNF] = BT * C;
    n[A_LNF_MEAN] = BT;
    n[A_LNF_RSTD] = BT;
    n[A_LOGITS] = BT * s->V; /* the oracle keeps only the V real columns */
    n[A_PROBS] = BT * s->V;
    n[A_LOSSES] = BT;
}

i64 ref_num_activations(int maxT, int V, int Vp, int L, int NH, int C, int B, int T) {
    ref_shape s = {maxT, V, Vp, L, NH, C};
    i64 n[NUM_ACTS], total = 0;
    act_counts(&s, B, T, n);
    for (int i = 0; i < NUM_ACTS; i++) total += n[i];
    return total;
}

/* ------------------------------------------------------------------------ */
/* layers                                                                    */
/* ------------------------------------------------------------------------ */

/* Encoder: the token-embedding row of each token plus the position-embedding
 * row of its position (InfoQ layer list, "encoder"). */
void ref_encoder_forward(double *out, const int *tok, const double *wte, const double *wpe,
                         int B, int T, int C) {
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            const double *we = wte + (i64)tok[b * T + t] * C;
            const double *pe = wpe + (i64)t * C;
            double *o = out + ((i64)b * T + t) * C;
            for (int c = 0; c < C; c++) o[c] = we[c] + pe[c];
        }
}

/* Encoder backward: every position adds its gradient row into the embedding
 * row of its token and into the row of its position; b outer, t inner. */
void ref_encoder_backward(double *dwte, double *dwpe, const double *dout, const int *tok,
                          int B, int T, int C) {
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            const double *d = dout + ((i64)b * T + t) * C;
            double *gw = dwte + (i64)tok[b * T + t] * C;
            double *gp = dwpe + (i64)t * C;
            for (int c = 0; c < C; c++) {
                gw[c] += d[c];
                gp[c] += d[c];
            }
        }
}

/* LayerNorm over the C channels of each of N rows: mean, biased variance,
 * rstd = 1/sqrt(var + 1e-5), then the affine map (GeekNews, "Triển khai các
 * lớp mạng nơ-ron": normalise mean and variance). */
void ref_layernorm_forward(double *out, double *mean, double *rstd, const double *inp,
                           const double *w, const double *bias, int N, int C) {
    const double eps = 1e-5;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < N; r++) {
        const double *x = inp + (i64)r * C;
        double m = 0.0;
        for (int c = 0; c < C; c++) m += x[c];
        m = m / C;
        double v = 0.0;
        for (int c = 0; c < C; c++) v += (x[c] - m) * (x[c] - m);
        v = v / C;
        double s = 1.0 / sqrt(v + eps);
        double *o = out + (i64)r * C;
        for (int c = 0; c < C; c++) o[c] = (x[c] - m) * s * w[c] + bias[c];
        mean[r] = m;
        rstd[r] = s;
    }
}

/* LayerNorm backward (chain rule through the definition above):
 * xhat = (x - mean) * rstd, g = dout * w,
 * dx += rstd * (g - mean_c(g) - xhat * mean_c(g * xhat)),
 * dw += sum_rows dout * xhat, db += sum_rows dout. */
void ref_layernorm_backward(double *dinp, double *dw, double *db, const double *dout,
                            const double *inp, const double *w, const double *mean,
                            const double *rstd, int N, int C) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < N; r++) {
        const double *x = inp + (i64)r * C;
        const double *dy = dout + (i64)r * C;
        double *dx = dinp + (i64)r * C;
        double g_mean = 0.0, gx_mean = 0.0;
        for (int c = 0; c < C; c++) {
            double xhat = (x[c] - mean[r]) * rstd[r];
            double g = dy[c] * w[c];
            g_mean += g;
            gx_mean += g * xhat;
        }
        g_mean /= C;
        gx_mean /= C;
        for (int c = 0; c < C; c++) {
            double xhat = (x[c] - mean[r]) * rstd[r];
            double g = dy[c] * w[c];
            dx[c] += rstd[r] * (g - g_mean - xhat * gx_mean);
        }
    }
    /* parameter grads: each channel sums over rows 0..N-1 in order */
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; c++) {
        double sw = 0.0, sb = 0.0;
        for (int r = 0; r < N; r++) {
            double xhat = (inp[(i64)r * C + c] - mean[r]) * rstd[r];
            sw += dout[(i64)r * C + c] * xhat;
            sb += dout[(i64)r * C + c];
        }
        dw[c] += sw;
        db[c] += sb;
    }
}

/* ------------------------------------------------------------------------ */
/* reduced-precision products                                                */
/* ------------------------------------------------------------------------ */

/* The QbitAI llm.c article ("手動實現每個層前向/反向傳播") names lower precision
 * (fp16 and below) as the next step for the trainer.  Reading taken here: in
 * that mode the operands of every linear-layer product (the qkv, projection,
 * MLP and head matmuls, forward and backward) are rounded to bfloat16 -- 8
 * significant bits, the exponent range of fp32 -- and the products are
 * accumulated at full precision; everything else (attention, LayerNorm,
 * softmax, GELU, bias sums, AdamW and the stored parameters) stays as it is. */

/* x rounded to the nearest value with 8 significant bits, ties to even. */
double ref_round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double m = frexp(x, &e);           /* x = m 2^e, 0.5 <= |m| < 1 */
    double r = rint(ldexp(m, 8));      /* 8 significant bits; rint rounds ties to even */
    return ldexp(r, e - 8);
}

static int ref_bf16_products = 0;

/* 0: products of the operands as given; 1: of their bfloat16 roundings. */
void ref_set_bf16_products(int on) { ref_bf16_products = on != 0; }

/* a copy of n operand values, rounded when the bfloat16 mode is on (NULL
 * when it is off: use the operand itself) */
static double *bf16_operand(const double *a, i64 n) {
    if (!ref_bf16_products) return NULL;
    double *c = malloc(sizeof(double) * (size_t)n);
    for (i64 i = 0; i < n; i++) c[i] = ref_round_bf16(a[i]);
    return c;
}

/* Linear: out[r][o] = bias[o] + sum_i inp[r][i] * W[o][i]  (W is OC x K,
 * row o holds the input weights of output o; bias may be NULL) -- GeekNews,
 * "Triển khai các lớp mạng nơ-ron": matmul, then the bias on every row. */
void ref_matmul_forward(double *out, const double *inp, const double *W, const double *bias,
                        int N, int K, int OC) {
    double *ri = bf16_operand(inp, (i64)N * K), *rw = bf16_operand(W, (i64)OC * K);
    if (ri) inp = ri;
    if (rw) W = rw;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < N; r++) {
        const double *x = inp + (i64)r * K;
        for (int o = 0; o < OC; o++) {
            const double *wr = W + (i64)o * K;
            double acc = 0.0;
            for (int i = 0; i < K; i++) acc += x[i] * wr[i];
            out[(i64)r * OC + o] = (bias ? bias[o] : 0.0) + acc;
        }
    }
    free(ri);
    free(rw);
}

/* Linear backward:
 *   dinp[r][i] += sum_o dout[r][o] * W[o][i]
 *   dW[o][i]   += sum_r dout[r][o] * inp[r][i]
 *   db[o]      += sum_r dout[r][o]          (db may be NULL)
 * Each sum runs over its index from 0 upward; the loops are nested so that
 * the innermost index is contiguous in memory, which does not change any sum. */
void ref_matmul_backward(double *dinp, double *dW, double *db, const double *dout,
                         const double *inp, const double *W, int N, int K, int OC) {
    /* operands of the two products (rounded in the bfloat16 mode); the bias
     * sum is no product and takes dout as given */
    double *rd = bf16_operand(dout, (i64)N * OC), *ri = bf16_operand(inp, (i64)N * K);
    double *rw = bf16_operand(W, (i64)OC * K);
    const double *pd = rd ? rd : dout, *pi = ri ? ri : inp, *pw = rw ? rw : W;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < N; r++) {
        double *dx = dinp + (i64)r * K;
        for (int o = 0; o < OC; o++) {
            double d = pd[(i64)r * OC + o];
            const double *wr = pw + (i64)o * K;
            for (int i = 0; i < K; i++) dx[i] += d * wr[i];
        }
    }
#pragma omp parallel for schedule(static)
    for (int o = 0; o < OC; o++) {
        double *gw = dW + (i64)o * K;
        double sb = 0.0;
        for (int r = 0; r < N; r++) {
            double d = pd[(i64)r * OC + o];
            const double *x = pi + (i64)r * K;
            for (int i = 0; i < K; i++) gw[i] += d * x[i];
            sb += dout[(i64)r * OC + o];
        }
        if (db) db[o] += sb;
    }
    free(rd);
    free(ri);
    free(rw);
}

/* Causal multi-head self-attention over qkv rows [q | k | v] (each C wide;
 * head h owns columns h*hd .. h*hd+hd-1 of each block).  For query t and key
 * u <= t (the lower triangle: a token sees itself and the past --
 * GeekNews, "Triển khai các lớp mạng nơ-ron" and "Phần lõi Transformer"):
 *   preatt[t][u] = (q_t . k_u) / sqrt(hd)
 *   att[t][u]    = exp(preatt[t][u] - max) / sum_{u' <= t} exp(preatt[t][u'] - max)
 *   out[t]       = sum_{u <= t} att[t][u] * v_u      (heads concatenated)
 * att[t][u > t] = 0; preatt[t][u > t] is set to 0 and has no meaning.
 * preatt and att are [B][NH][T][T]. */
void ref_attention_forward(double *out, double *preatt, double *att, const double *qkv,
                           int B, int T, int C, int NH) {
    int hd = C / NH;
    double scale = 1.0 / sqrt((double)hd);
    i64 C3 = 3 * (i64)C;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++) {
            for (int t = 0; t < T; t++) {
                const double *q = qkv + ((i64)b * T + t) * C3 + (i64)h * hd;
                double *pre = preatt + (((i64)b * NH + h) * T + t) * T;
                double *a = att + (((i64)b * NH + h) * T + t) * T;
                double mx = -INFINITY;
                for (int u = 0; u <= t; u++) {
                    const double *k = qkv + ((i64)b * T + u) * C3 + C + (i64)h * hd;
                    double s = 0.0;
                    for (int d = 0; d < hd; d++) s += q[d] * k[d];
                    s *= scale;
                    pre[u] = s;
                    if (s > mx) mx = s;
                }
                double sum = 0.0;
                for (int u = 0; u <= t; u++) {
                    a[u] = exp(pre[u] - mx);
                    sum += a[u];
                }
                for (int u = 0; u <= t; u++) a[u] /= sum;
                for (int u = t + 1; u < T; u++) {
                    a[u] = 0.0;
                    pre[u] = 0.0;
                }
                double *o = out + ((i64)b * T + t) * C + (i64)h * hd;
                for (int d = 0; d < hd; d++) {
                    double acc = 0.0;
                    for (int u = 0; u <= t; u++) {
                        const double *v = qkv + ((i64)b * T + u) * C3 + 2 * (i64)C + (i64)h * hd;
                        acc += a[u] * v[d];
                    }
                    o[d] = acc;
                }
            }
        }
}

/* Attention backward, by the chain rule through the forward above:
 *   datt[t][u]    = dout_t . v_u                                  (u <= t)
 *   dv_u         += att[t][u] * dout_t
 *   dpreatt[t][u] = att[t][u] * (datt[t][u] - sum_{u'<=t} att[t][u'] datt[t][u'])
 *   dq_t         += dpreatt[t][u] * k_u / sqrt(hd)
 *   dk_u         += dpreatt[t][u] * q_t / sqrt(hd)
 * dqkv accumulates; dpreatt and datt ([B][NH][T][T]) are overwritten (their
 * entries above the diagonal are set to 0). */
void ref_attention_backward(double *dqkv, double *dpreatt, double *datt, const double *dout,
                            const double *qkv, const double *att, int B, int T, int C,
                            int NH) {
    int hd = C / NH;
    double scale = 1.0 / sqrt((double)hd);
    i64 C3 = 3 * (i64)C;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++) {
            for (int t = 0; t < T; t++) {
                const double *a = att + (((i64)b * NH + h) * T + t) * T;
                double *da = datt + (((i64)b * NH + h) * T + t) * T;
                double *dp = dpreatt + (((i64)b * NH + h) * T + t) * T;
                const double *dy = dout + ((i64)b * T + t) * C + (i64)h * hd;
                for (int u = 0; u <= t; u++) {
                    const double *v = qkv + ((i64)b * T + u) * C3 + 2 * (i64)C + (i64)h * hd;
                    double *dv = dqkv + ((i64)b * T + u) * C3 + 2 * (i64)C + (i64)h * hd;
                    double s = 0.0;
                    for (int d = 0; d < hd; d++) s += dy[d] * v[d];
                    da[u] = s;
                    for (int d = 0; d < hd; d++) dv[d] += a[u] * dy[d];
                }
                double dot = 0.0;
                for (int u = 0; u <= t; u++) dot += a[u] * da[u];
                for (int u = 0; u <= t; u++) dp[u] = a[u] * (da[u] - dot);
                for (int u = t + 1; u < T; u++) {
                    da[u] = 0.0;
                    dp[u] = 0.0;
                }
                const double *q = qkv + ((i64)b * T + t) * C3 + (i64)h * hd;
                double *dq = dqkv + ((i64)b * T + t) * C3 + (i64)h * hd;
                for (int u = 0; u <= t; u++) {
                    const double *k = qkv + ((i64)b * T + u) * C3 + C + (i64)h * hd;
                    double *dk = dqkv + ((i64)b * T + u) * C3 + C + (i64)h * hd;
                    for (int d = 0; d < hd; d++) {
                        dq[d] += dp[u] * k[d] * scale;
                        dk[d] += dp[u] * q[d] * scale;
                    }
                }
            }
        }
}

/* tanh-approximate GELU, 0.5 x (1 + tanh(k (x + 0.044715 x^3))), k = sqrt(2/pi)
 * (GeekNews comment thread: the GELU macro with .7978845 and .044715). */
static double gelu_k(void) { return sqrt(2.0 / M_PI); }

void ref_gelu_forward(double *out, const double *inp, i64 n) {
    double k = gelu_k();
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; i++) {
        double x = inp[i];
        out[i] = 0.5 * x * (1.0 + tanh(k * (x + 0.044715 * x * x * x)));
    }
}

/* d/dx of the above: 0.5 (1 + tanh u) + 0.5 x (1 - tanh^2 u) k (1 + 3 * 0.044715 x^2),
 * u = k (x + 0.044715 x^3).  dinp accumulates. */
void ref_gelu_backward(double *dinp, const double *inp, const double *dout, i64 n) {
    double k = gelu_k();
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; i++) {
        double x = inp[i];
        double u = k * (x + 0.044715 * x * x * x);
        double th = tanh(u);
        double dudx = k * (1.0 + 3.0 * 0.044715 * x * x);
        double g = 0.5 * (1.0 + th) + 0.5 * x * (1.0 - th * th) * dudx;
        dinp[i] += g * dout[i];
    }
}

/* Residual connection: out = a + b. */
void ref_residual_forward(double *out, const double *a, const double *b, i64 n) {
    for (i64 i = 0; i < n; i++) out[i] = a[i] + b[i];
}

/* Softmax over the V real columns of each logits row, then cross-entropy
 * against the target: losses[r] = log(sum_v exp(z_v - max)) + max - z[target].
 * logits rows are `ld` wide (ld >= V); only columns < V take part. */
void ref_softmax_crossentropy_forward(double *losses, double *probs, const double *logits,
                                      const int *targets, int N, int V, int ld) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < N; r++) {
        const double *z = logits + (i64)r * ld;
        double *p = probs + (i64)r * V;
        double mx = -INFINITY;
        for (int v = 0; v < V; v++)
            if (z[v] > mx) mx = z[v];
        double sum = 0.0;
        for (int v = 0; v < V; v++) sum += exp(z[v] - mx);
        for (int v = 0; v < V; v++) p[v] = exp(z[v] - mx) / sum;
        if (targets) losses[r] = log(sum) + mx - z[targets[r]];
    }
}

/* Gradient of mean(losses) w.r.t. the logits: (probs - onehot(target)) / N.
 * dlogits rows are `ld` wide; columns >= V are set to 0. */
void ref_crossentropy_softmax_backward(double *dlogits, const double *probs,
                                       const int *targets, int N, int V, int ld) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < N; r++) {
        double *d = dlogits + (i64)r * ld;
        const double *p = probs + (i64)r * V;
        for (int v = 0; v < V; v++) d[v] = (p[v] - (v == targets[r] ? 1.0 : 0.0)) / N;
        for (int v = V; v < ld; v++) d[v] = 0.0;
    }
}

/* AdamW over n elements, t >= 1 (InfoQ run log: Adam at lr 1e-4; decoupled
 * weight decay):
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2
 *   mhat = m / (1 - b1^t); vhat = v / (1 - b2^t)
 *   theta -= lr * (mhat / (sqrt(vhat) + eps) + wd * theta) */
void ref_adamw(double *params, const double *grads, double *m, double *v, i64 n, double lr,
               double b1, double b2, double eps, double wd, int t) {
    double c1 = 1.0 - pow(b1, t), c2 = 1.0 - pow(b2, t);
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; i++) {
        double g = grads[i];
        m[i] = b1 * m[i] + (1.0 - b1) * g;
        v[i] = b2 * v[i] + (1.0 - b2) * g * g;
        double mhat = m[i] / c1, vhat = v[i] / c2;
        params[i] -= lr * (mhat / (sqrt(vhat) + eps) + wd * params[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* the whole model                                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
    ref_shape s;
    int B, T;
    i64 poff[REF_NUM_PARAM_TENSORS];
    i64 aoff[NUM_ACTS], acount[NUM_ACTS];
    double *acts;       /* the 23 saved tensors, one allocation  */
    double *grad_acts;  /* same shape as acts, for the backward   */
    double *dlogits;    /* [B*T][V]                               */
    int *inputs, *targets;
    int have_targets;
} ref_model;

ref_model *ref_create(int maxT, int V, int Vp, int L, int NH, int C, int B, int T) {
    if (maxT <= 0 || V <= 0 || Vp < V || L <= 0 || NH <= 0 || C <= 0 || C % NH || B <= 0 ||
        T <= 0 || T > maxT)
        return NULL;
    ref_model *M = (ref_model *)calloc(1, sizeof(ref_model));
    ref_shape s = {maxT, V, Vp, L, NH, C};
    M->s = s;
    M->B = B;
    M->T = T;
    i64 pn[REF_NUM_PARAM_TENSORS], off = 0;
    param_counts(&s, pn);
    for (int i = 0; i < REF_NUM_PARAM_TENSORS; i++) {
        M->poff[i] = off;
        off += pn[i];
    }
    act_counts(&s, B, T, M->acount);
    off = 0;
    for (int i = 0; i < NUM_ACTS; i++) {
        M->aoff[i] = off;
        off += M->acount[i];
    }
    M->acts = (double *)calloc((size_t)off, sizeof(double));
    M->grad_acts = (double *)calloc((size_t)off, sizeof(double));
    M->dlogits = (double *)calloc((size_t)B * T * V, sizeof(double));
    M->inputs = (int *)calloc((size_t)B * T, sizeof(int));
    M->targets = (int *)calloc((size_t)B * T, sizeof(int));
    if (!M->acts || !M->grad_acts || !M->dlogits || !M->inputs || !M->targets) {
        free(M->acts);
        free(M->grad_acts);
        free(M->dlogits);
        free(M->inputs);
        free(M->targets);
        free(M);
        return NULL;
    }
    return M;
}

void ref_destroy(ref_model *M) {
    if (!M) return;
    free(M->acts);
    free(M->grad_acts);
    free(M->dlogits);
    free(M->inputs);
    free(M->targets);
    free(M);
}

#define ACT(M, id) ((M)->acts + (M)->aoff[id])
#define GACT(M, id) ((M)->grad_acts + (M)->aoff[id])
#define PAR(M, P, id) ((P) + (M)->poff[id])

/* Forward pass (GeekNews, "Phần lõi Transformer"): encoder; per layer
 * LN -> qkv linear -> causal attention -> projection + residual -> LN ->
 * fc linear -> GELU -> projection + residual; final LN; logits = lnf . wte^T
 * over v < V; softmax cross-entropy.  Returns the mean loss when targets is
 * given, else NAN.  Returns -1.0 / sets nothing for an out-of-range token. */
double ref_forward(ref_model *M, const double *params, const int *inputs, const int *targets) {
    int B = M->B, T = M->T, C = M->s.C, L = M->s.L, NH = M->s.NH, V = M->s.V;
    i64 BT = (i64)B * T, BTC = BT * C;
    for (i64 i = 0; i < BT; i++) {
        if (inputs[i] < 0 || inputs[i] >= V) return -1.0;
        if (targets && (targets[i] < 0 || targets[i] >= V)) return -1.0;
    }
    memcpy(M->inputs, inputs, sizeof(int) * BT);
    if (targets) memcpy(M->targets, targets, sizeof(int) * BT);
    M->have_targets = targets != NULL;

    ref_encoder_forward(ACT(M, A_ENCODED), inputs, PAR(M, params, 0), PAR(M, params, 1), B, T, C);
    for (int l = 0; l < L; l++) {
        const double *res = l == 0 ? ACT(M, A_ENCODED) : ACT(M, A_RESIDUAL3) + (i64)(l - 1) * BTC;
        const double *ln1w = PAR(M, params, 2) + (i64)l * C, *ln1b = PAR(M, params, 3) + (i64)l * C;
        const double *qkvw = PAR(M, params, 4) + (i64)l * 3 * C * C;
        const double *qkvb = PAR(M, params, 5) + (i64)l * 3 * C;
        const double *aw = PAR(M, params, 6) + (i64)l * C * C, *ab = PAR(M, params, 7) + (i64)l * C;
        const double *ln2w = PAR(M, params, 8) + (i64)l * C, *ln2b = PAR(M, params, 9) + (i64)l * C;
        const double *fw = PAR(M, params, 10) + (i64)l * 4 * C * C;
        const double *fb = PAR(M, params, 11) + (i64)l * 4 * C;
        const double *pw = PAR(M, params, 12) + (i64)l * 4 * C * C;
        const double *pb = PAR(M, params, 13) + (i64)l * C;
        double *ln1 = ACT(M, A_LN1) + l * BTC, *ln1m = ACT(M, A_LN1_MEAN) + l * BT;
        double *ln1r = ACT(M, A_LN1_RSTD) + l * BT, *qkv = ACT(M, A_QKV) + l * 3 * BTC;
        double *atty = ACT(M, A_ATTY) + l * BTC;
        double *pre = ACT(M, A_PREATT) + (i64)l * B * NH * T * T;
        double *att = ACT(M, A_ATT) + (i64)l * B * NH * T * T;
        double *ap = ACT(M, A_ATTPROJ) + l * BTC, *r2 = ACT(M, A_RESIDUAL2) + l * BTC;
        double *ln2 = ACT(M, A_LN2) + l * BTC, *ln2m = ACT(M, A_LN2_MEAN) + l * BT;
        double *ln2r = ACT(M, A_LN2_RSTD) + l * BT;
        double *fch = ACT(M, A_FCH) + l * 4 * BTC, *fchg = ACT(M, A_FCH_GELU) + l * 4 * BTC;
        double *fp = ACT(M, A_FCPROJ) + l * BTC, *r3 = ACT(M, A_RESIDUAL3) + l * BTC;

        ref_layernorm_forward(ln1, ln1m, ln1r, res, ln1w, ln1b, (int)BT, C);
        ref_matmul_forward(qkv, ln1, qkvw, qkvb, (int)BT, C, 3 * C);
        ref_attention_forward(atty, pre, att, qkv, B, T, C, NH);
        ref_matmul_forward(ap, atty, aw, ab, (int)BT, C, C);
        ref_residual_forward(r2, res, ap, BTC);
        ref_layernorm_forward(ln2, ln2m, ln2r, r2, ln2w, ln2b, (int)BT, C);
        ref_matmul_forward(fch, ln2, fw, fb, (int)BT, C, 4 * C);
        ref_gelu_forward(fchg, fch, 4 * BTC);
        ref_matmul_forward(fp, fchg, pw, pb, (int)BT, 4 * C, C);
        ref_residual_forward(r3, r2, fp, BTC);
    }
    const double *last = ACT(M, A_RESIDUAL3) + (i64)(L - 1) * BTC;
    ref_layernorm_forward(ACT(M, A_LNF), ACT(M, A_LNF_MEAN), ACT(M, A_LNF_RSTD), last,
                          PAR(M, params, 14), PAR(M, params, 15), (int)BT, C);
    /* tied head: the first V rows of wte, no bias (GeekNews, "Phần lõi Transformer") */
    ref_matmul_forward(ACT(M, A_LOGITS), ACT(M, A_LNF), PAR(M, params, 0), NULL, (int)BT, C, V);
    ref_softmax_crossentropy_forward(ACT(M, A_LOSSES), ACT(M, A_PROBS), ACT(M, A_LOGITS),
                                     targets, (int)BT, V, V);
    if (!targets) return NAN;
    double loss = 0.0;
    for (i64 i = 0; i < BT; i++) loss += ACT(M, A_LOSSES)[i];
    return loss / BT;
}

/* Backward pass of the mean loss, accumulating into grads (same layout as
 * params).  Needs a preceding forward with targets; returns 0, or -1. */
int ref_backward(ref_model *M, const double *params, double *grads) {
    if (!M->have_targets) return -1;
    int B = M->B, T = M->T, C = M->s.C, L = M->s.L, NH = M->s.NH, V = M->s.V;
    i64 BT = (i64)B * T, BTC = BT * C;
    i64 total = 0;
    for (int i = 0; i < NUM_ACTS; i++) total += M->acount[i];
    memset(M->grad_acts, 0, sizeof(double) * (size_t)total);

    ref_crossentropy_softmax_backward(M->dlogits, ACT(M, A_PROBS), M->targets, (int)BT, V, V);
    ref_matmul_backward(GACT(M, A_LNF), PAR(M, grads, 0), NULL, M->dlogits, ACT(M, A_LNF),
                        PAR(M, params, 0), (int)BT, C, V);
    double *dlast = GACT(M, A_RESIDUAL3) + (i64)(L - 1) * BTC;
    ref_layernorm_backward(dlast, PAR(M, grads, 14), PAR(M, grads, 15), GACT(M, A_LNF),
                           ACT(M, A_RESIDUAL3) + (i64)(L - 1) * BTC, PAR(M, params, 14),
                           ACT(M, A_LNF_MEAN), ACT(M, A_LNF_RSTD), (int)BT, C);
    for (int l = L - 1; l >= 0; l--) {
        const double *res = l == 0 ? ACT(M, A_ENCODED) : ACT(M, A_RESIDUAL3) + (i64)(l - 1) * BTC;
        double *dres = l == 0 ? GACT(M, A_ENCODED) : GACT(M, A_RESIDUAL3) + (i64)(l - 1) * BTC;
        const double *ln1w = PAR(M, params, 2) + (i64)l * C;
        const double *qkvw = PAR(M, params, 4) + (i64)l * 3 * C * C;
        const double *aw = PAR(M, params, 6) + (i64)l * C * C;
        const double *ln2w = PAR(M, params, 8) + (i64)l * C;
        const double *fw = PAR(M, params, 10) + (i64)l * 4 * C * C;
        const double *pw = PAR(M, params, 12) + (i64)l * 4 * C * C;
        double *g_ln1w = PAR(M, grads, 2) + (i64)l * C, *g_ln1b = PAR(M, grads, 3) + (i64)l * C;
        double *g_qkvw = PAR(M, grads, 4) + (i64)l * 3 * C * C;
        double *g_qkvb = PAR(M, grads, 5) + (i64)l * 3 * C;
        double *g_aw = PAR(M, grads, 6) + (i64)l * C * C, *g_ab = PAR(M, grads, 7) + (i64)l * C;
        double *g_ln2w = PAR(M, grads, 8) + (i64)l * C, *g_ln2b = PAR(M, grads, 9) + (i64)l * C;
        double *g_fw = PAR(M, grads, 10) + (i64)l * 4 * C * C;
        double *g_fb = PAR(M, grads, 11) + (i64)l * 4 * C;
        double *g_pw = PAR(M, grads, 12) + (i64)l * 4 * C * C;
        double *g_pb = PAR(M, grads, 13) + (i64)l * C;

        const double *ln1 = ACT(M, A_LN1) + l * BTC, *ln1m = ACT(M, A_LN1_MEAN) + l * BT;
        const double *ln1r = ACT(M, A_LN1_RSTD) + l * BT, *qkv = ACT(M, A_QKV) + l * 3 * BTC;
        const double *atty = ACT(M, A_ATTY) + l * BTC;
        const double *att = ACT(M, A_ATT) + (i64)l * B * NH * T * T;
        const double *r2 = ACT(M, A_RESIDUAL2) + l * BTC;
        const double *ln2 = ACT(M, A_LN2) + l * BTC, *ln2m = ACT(M, A_LN2_MEAN) + l * BT;
        const double *ln2r = ACT(M, A_LN2_RSTD) + l * BT;
        const double *fch = ACT(M, A_FCH) + l * 4 * BTC, *fchg = ACT(M, A_FCH_GELU) + l * 4 * BTC;

        double *d_ln1 = GACT(M, A_LN1) + l * BTC, *d_qkv = GACT(M, A_QKV) + l * 3 * BTC;
        double *d_atty = GACT(M, A_ATTY) + l * BTC;
        double *d_pre = GACT(M, A_PREATT) + (i64)l * B * NH * T * T;
        double *d_att = GACT(M, A_ATT) + (i64)l * B * NH * T * T;
        double *d_ap = GACT(M, A_ATTPROJ) + l * BTC, *d_r2 = GACT(M, A_RESIDUAL2) + l * BTC;
        double *d_ln2 = GACT(M, A_LN2) + l * BTC;
        double *d_fch = GACT(M, A_FCH) + l * 4 * BTC, *d_fchg = GACT(M, A_FCH_GELU) + l * 4 * BTC;
        double *d_fp = GACT(M, A_FCPROJ) + l * BTC, *d_r3 = GACT(M, A_RESIDUAL3) + l * BTC;

        /* residual3 = residual2 + fcproj: its gradient reaches both terms */
        for (i64 i = 0; i < BTC; i++) {
            d_r2[i] += d_r3[i];
            d_fp[i] += d_r3[i];
        }
        ref_matmul_backward(d_fchg, g_pw, g_pb, d_fp, fchg, pw, (int)BT, 4 * C, C);
        ref_gelu_backward(d_fch, fch, d_fchg, 4 * BTC);
        ref_matmul_backward(d_ln2, g_fw, g_fb, d_fch, ln2, fw, (int)BT, C, 4 * C);
        ref_layernorm_backward(d_r2, g_ln2w, g_ln2b, d_ln2, r2, ln2w, ln2m, ln2r, (int)BT, C);
        /* residual2 = residual + attproj */
        for (i64 i = 0; i < BTC; i++) {
            dres[i] += d_r2[i];
            d_ap[i] += d_r2[i];
        }
        ref_matmul_backward(d_atty, g_aw, g_ab, d_ap, atty, aw, (int)BT, C, C);
        ref_attention_backward(d_qkv, d_pre, d_att, d_atty, qkv, att, B, T, C, NH);
        ref_matmul_backward(d_ln1, g_qkvw, g_qkvb, d_qkv, ln1, qkvw, (int)BT, C, 3 * C);
        ref_layernorm_backward(dres, g_ln1w, g_ln1b, d_ln1, res, ln1w, ln1m, ln1r, (int)BT, C);
    }
    ref_encoder_backward(PAR(M, grads, 0), PAR(M, grads, 1), GACT(M, A_ENCODED), M->inputs, B, T,
                         C);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* decoding with a key/value cache                                          */
/* ------------------------------------------------------------------------ */

/* The next token from one row of logits z[0..V-1] (GeekNews, "Cách KV caching
 * hoạt động": generation picks one token per step; the InfoQ article's run
 * prints the sampled token ids).  coin < 0: the most probable token (the
 * lowest index among equal maxima).  Otherwise, with p = softmax(z) (max
 * subtracted), the first v whose cumulative probability p_0 + ... + p_v
 * exceeds coin; coin is a uniform draw in [0, 1) supplied by the caller. */
int ref_sample(const double *z, int V, double coin) {
    int best = 0;
    for (int v = 1; v < V; v++)
        if (z[v] > z[best]) best = v;
    if (coin < 0.0) return best;
    double sum = 0.0;
    for (int v = 0; v < V; v++) sum += exp(z[v] - z[best]);
    double cum = 0.0;
    for (int v = 0; v < V; v++) {
        cum += exp(z[v] - z[best]) / sum;
        if (cum > coin) return v;
    }
    return V - 1;
}

/* One decoding step (GeekNews, "Cách KV caching hoạt động": the keys and
 * values of the tokens already processed are kept, so a new token needs only
 * its own row through every layer; "Phép nhân ma trận nhanh": only the new
 * rows of a product are multiplied).  For each sequence b, tokens[b] is the
 * token at position pos (0 <= pos < T); rows (b, u < pos) of the saved qkv
 * activations must hold the keys and values of the earlier positions, from
 * ref_forward over them or from earlier decode steps.  Row (b, pos) goes
 * through the same layers as in ref_forward (encoder, then per layer LN ->
 * qkv -> attention over u <= pos -> projection + residual -> LN -> fc ->
 * GELU -> projection + residual, final LN, tied head over v < V).  It writes
 * row (b, pos) of every layer's qkv (the cache) and of the logits, and
 * next[b] = ref_sample(logits row, coins ? coins[b] : -1).  Returns 0, or -1
 * for a bad position or token. */
int ref_decode_step(ref_model *M, const double *params, const int *tokens, int pos, const double *coins,
                    int *next) {
    int B = M->B, T = M->T, C = M->s.C, L = M->s.L, NH = M->s.NH, V = M->s.V;
    if (pos < 0 || pos >= T) return -1;
    for (int b = 0; b < B; b++)
        if (tokens[b] < 0 || tokens[b] >= V) return -1;
    int hd = C / NH;
    i64 BT = (i64)B * T, BTC = BT * C, C3 = 3 * (i64)C;
    double scale = 1.0 / sqrt((double)hd);
    double *x = malloc(sizeof(double) * C), *ln = malloc(sizeof(double) * C);
    double *atty = malloc(sizeof(double) * C), *tmp = malloc(sizeof(double) * C);
    double *h = malloc(sizeof(double) * 4 * C), *g = malloc(sizeof(double) * 4 * C);
    double *s = malloc(sizeof(double) * (pos + 1)), mean, rstd;
    for (int b = 0; b < B; b++) {
        i64 row = (i64)b * T + pos;
        ref_encoder_forward(x, &tokens[b], PAR(M, params, 0), PAR(M, params, 1) + (i64)pos * C, 1, 1, C);
        for (int l = 0; l < L; l++) {
            double *qkv = ACT(M, A_QKV) + l * 3 * BTC; /* this layer's cache */
            ref_layernorm_forward(ln, &mean, &rstd, x, PAR(M, params, 2) + (i64)l * C,
                                  PAR(M, params, 3) + (i64)l * C, 1, C);
            ref_matmul_forward(qkv + row * C3, ln, PAR(M, params, 4) + (i64)l * 3 * C * C,
                               PAR(M, params, 5) + (i64)l * 3 * C, 1, C, 3 * C);
            /* the new query against the cached keys u <= pos, per head */
            for (int hh = 0; hh < NH; hh++) {
                const double *q = qkv + row * C3 + (i64)hh * hd;
                double mx = -INFINITY;
                for (int u = 0; u <= pos; u++) {
                    const double *k = qkv + ((i64)b * T + u) * C3 + C + (i64)hh * hd;
                    double d = 0.0;
                    for (int e = 0; e < hd; e++) d += q[e] * k[e];
                    s[u] = d * scale;
                    if (s[u] > mx) mx = s[u];
                }
                double sum = 0.0;
                for (int u = 0; u <= pos; u++) {
                    s[u] = exp(s[u] - mx);
                    sum += s[u];
                }
                for (int e = 0; e < hd; e++) {
                    double y = 0.0;
                    for (int u = 0; u <= pos; u++)
                        y += s[u] / sum * qkv[((i64)b * T + u) * C3 + 2 * C + (i64)hh * hd + e];
                    atty[(i64)hh * hd + e] = y;
                }
            }
            ref_matmul_forward(tmp, atty, PAR(M, params, 6) + (i64)l * C * C, PAR(M, params, 7) + (i64)l * C, 1,
                               C, C);
            ref_residual_forward(x, x, tmp, C);
            ref_layernorm_forward(ln, &mean, &rstd, x, PAR(M, params, 8) + (i64)l * C,
                                  PAR(M, params, 9) + (i64)l * C, 1, C);
            ref_matmul_forward(h, ln, PAR(M, params, 10) + (i64)l * 4 * C * C, PAR(M, params, 11) + (i64)l * 4 * C,
                               1, C, 4 * C);
            ref_gelu_forward(g, h, 4 * C);
            ref_matmul_forward(tmp, g, PAR(M, params, 12) + (i64)l * 4 * C * C, PAR(M, params, 13) + (i64)l * C, 1,
                               4 * C, C);
            ref_residual_forward(x, x, tmp, C);
        }
        ref_layernorm_forward(ln, &mean, &rstd, x, PAR(M, params, 14), PAR(M, params, 15), 1, C);
        double *z = ACT(M, A_LOGITS) + row * V;
        ref_matmul_forward(z, ln, PAR(M, params, 0), NULL, 1, C, V);
        next[b] = ref_sample(z, V, coins ? coins[b] : -1.0);
    }
    free(x); free(ln); free(atty); free(tmp); free(h); free(g); free(s);
    M->have_targets = 0; /* the saved activations no longer describe one forward */
    return 0;
}

/* Copy out a saved activation (by name) or its gradient; returns the count
 * copied, or -1 for an unknown name or a short buffer. */
i64 ref_get(const ref_model *M, const char *name, int grad, double *out, i64 n) {
    for (int i = 0; i < NUM_ACTS; i++)
        if (strcmp(name, ref_act_names[i]) == 0) {
            if (n < M->acount[i]) return -1;
            memcpy(out, (grad ? M->grad_acts : M->acts) + M->aoff[i],
                   sizeof(double) * (size_t)M->acount[i]);
            return M->acount[i];
        }
    if (strcmp(name, "dlogits") == 0) {
        i64 cnt = (i64)M->B * M->T * M->s.V;
        if (n < cnt) return -1;
        memcpy(out, M->dlogits, sizeof(double) * (size_t)cnt);
        return cnt;
    }
    return -1;
}

i64 ref_act_count(const ref_model *M, const char *name) {
    for (int i = 0; i < NUM_ACTS; i++)
        if (strcmp(name, ref_act_names[i]) == 0) return M->acount[i];
    if (strcmp(name, "dlogits") == 0) return (i64)M->B * M->T * M->s.V;
    return -1;
}

int ref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
