/*
 * gpt2_kernels.h -- kernel-level entry points of libgpt2mi, for testing and
 * timing one step of the training path in isolation, at any shape.  They run
 * the same kernels, with the same launch planning, that gpt2_forward /
 * gpt2_backward / gpt2_update run.
 *
 * All pointers are DEVICE pointers (fp32 row-major unless noted, int32 ids),
 * 16-byte aligned; `stream` is a hipStream_t (NULL = null stream).  Calls are
 * asynchronous and return gpt2_status (GPT2_EINVAL for shapes a kernel cannot
 * take, GPT2_EDEVICE for a launch failure; message in gpt2_last_error(NULL)).
 * Sizes must be multiples of 4 where a row is read with 16-byte loads (C, K,
 * OC, T, Vp).  Where a call needs scratch it takes `work` with the float
 * count returned by the matching *_work function.
 */
#ifndef GPT2_MI_KERNELS_H
#define GPT2_MI_KERNELS_H

#include <stddef.h>
#include <stdint.h>

#include "gpt2.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Linear layer forward (GeekNews 3000-byte GPT-2 page, section on the layers:
 * matmul, then the bias on every row): out[N][OC] = inp[N][K] W[OC][K]^T (+ bias[OC]). */
gpt2_status gpt2k_linear_forward(float *out, const float *inp, const float *W, const float *bias, int N, int K,
                                 int OC, void *stream);

/* The same with the precision of the products given: GPT2_FP32, or GPT2_BF16
 * (operands rounded to bfloat16 for the matrix unit, fp32 accumulation; see
 * gpt2_set_matmul_precision). */
gpt2_status gpt2k_linear_forward_prec(float *out, const float *inp, const float *W, const float *bias, int N, int K,
                                      int OC, int precision, void *stream);

/* Linear layer backward: dinp[N][K] = dout W (overwritten; may be NULL to skip),
 * dW[OC][K] += dout^T inp, dbias[OC] += column sums of dout (may be NULL). */
size_t gpt2k_linear_backward_work(int N, int K, int OC);
gpt2_status gpt2k_linear_backward(float *dinp, float *dW, float *dbias, const float *dout, const float *inp,
                                  const float *W, int N, int K, int OC, float *work, void *stream);
/* The same with the precision of the two products given (the bias gradient,
 * a plain column sum of dout, is fp32 in both). */
gpt2_status gpt2k_linear_backward_prec(float *dinp, float *dW, float *dbias, const float *dout, const float *inp,
                                       const float *W, int N, int K, int OC, float *work, int precision,
                                       void *stream);

/* LayerNorm over rows of C (mean, biased variance, eps 1e-5, affine). */
gpt2_status gpt2k_layernorm_forward(float *out, float *mean, float *rstd, const float *inp, const float *w,
                                    const float *b, int N, int C, void *stream);
/* dinp = (accumulate ? dinp + : ) LayerNorm input gradient; dw, db += parameter gradients. */
size_t gpt2k_layernorm_backward_work(int N, int C);
gpt2_status gpt2k_layernorm_backward(float *dinp, float *dw, float *db, const float *dout, const float *inp,
                                     const float *w, const float *mean, const float *rstd, int N, int C,
                                     int accumulate, float *work, void *stream);

/* Causal multi-head attention over qkv[B][T][3C] (q | k | v, heads of C/NH),
 * with the score matrices materialised (any head dimension that is a
 * multiple of 4; T a multiple of 4): att[B][NH][T][T] = softmax probabilities (zero above the diagonal up to the
 * next multiple of 128 columns), atty[B][T][C] = heads concatenated. */
gpt2_status gpt2k_attention_forward(float *atty, float *att, const float *qkv, int B, int T, int C, int NH,
                                    void *stream);
/* dqkv[B][T][3C] = gradient of the forward above (overwritten) given datty;
 * work holds B*NH*T*T floats (the score gradient). */
size_t gpt2k_attention_backward_work(int B, int T, int C, int NH);
gpt2_status gpt2k_attention_backward(float *dqkv, const float *datty, const float *qkv, const float *att, int B,
                                     int T, int C, int NH, float *work, void *stream);

/* The same attention fused (the path gpt2_forward / gpt2_backward take when
 * the head dimension is 16, 32 or 64): the forward keeps no T x T matrix; it
 * writes atty and lse[B][NH][T] (log-sum-exp of each query's scaled scores).
 * The backward recomputes the probabilities from them, computes dk and dv,
 * stores ds = p (dp - D) for every causal (t, u) in `work`, and finishes dq
 * as a causal GEMM over ds; it overwrites dqkv.  Long causal rows are split
 * over workgroups (forward: chunks of at most 256 keys; dk/dv: equal ranges of
 * the (key block, query block) iterations over the resident workgroups) and
 * their partial results merged in a fixed order through `work`
 * (gpt2k_flash_attention_work floats, B*NH*T*Tp of them for ds, Tp = T
 * rounded up to a multiple of 4; the same size serves both calls).  Any
 * 1 <= T <= 1024.  GPT2_EINVAL for other head dimensions. */
size_t gpt2k_flash_attention_work(int B, int T, int C, int NH);
gpt2_status gpt2k_flash_attention_forward(float *atty, float *lse, const float *qkv, int B, int T, int C, int NH,
                                          float *work, void *stream);
gpt2_status gpt2k_flash_attention_backward(float *dqkv, const float *datty, const float *qkv, const float *atty,
                                           const float *lse, int B, int T, int C, int NH, float *work,
                                           void *stream);

/* tanh-GELU forward / backward (dinp = dout * gelu'(inp)), n % 4 == 0. */
gpt2_status gpt2k_gelu_forward(float *out, const float *inp, size_t n, void *stream);
gpt2_status gpt2k_gelu_backward(float *dinp, const float *inp, const float *dout, size_t n, void *stream);

/* Fused softmax cross-entropy over logits[BT][Vp] (first V columns real):
 * losses[BT], mean loss in loss[0], logits <- (softmax - onehot(target)) / BT. */
gpt2_status gpt2k_crossentropy(float *logits, float *losses, float *loss, const int32_t *targets, int BT, int V,
                               int Vp, void *stream);

/* Encoder: out[B][T][C] = wte[ids] + wpe[t].  Backward: dwte[id] += rows of
 * dout with that id, dwpe[t] += sum over b.  The backward needs the position
 * order computed by gpt2k_token_order (order: BT int32s, the positions
 * sorted by (id, position); err_flag |= 1 for an id, 2 for a target outside
 * [0, V); work: gpt2k_token_order_work(BT) int32s, 8-byte aligned, may be
 * NULL when that is 0) and gpt2k_encoder_backward_work floats of `work`
 * (segment sums). */
gpt2_status gpt2k_encoder_forward(float *out, const int32_t *ids, const float *wte, const float *wpe, int B, int T,
                                  int C, int V, void *stream);
size_t gpt2k_token_order_work(int BT);
gpt2_status gpt2k_token_order(int32_t *order, int32_t *err_flag, const int32_t *ids, const int32_t *targets,
                              int BT, int V, int32_t *work, void *stream);
size_t gpt2k_encoder_backward_work(int B, int T, int C);
gpt2_status gpt2k_encoder_backward(float *dwte, float *dwpe, const float *dout, const int32_t *ids,
                                   const int32_t *order, int B, int T, int C, int V, float *work, void *stream);

/* AdamW over n floats (n % 4 == 0), t >= 1; same update as gpt2_update. */
gpt2_status gpt2k_adamw(float *params, const float *grads, float *m, float *v, size_t n, float lr, float beta1,
                        float beta2, float eps, float weight_decay, int t, void *stream);

/* LayerNorm backward that allocates nothing, for callers that cannot call
 * hipMalloc or be handed a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, kernels
 * and results as gpt2k_layernorm_backward with dw and db given, but the
 * partial column sums of dw and db live in a static device array of
 * GPT2K_NOALLOC_SCRATCH_FLOATS floats (8 MiB) that each GPU holds from the
 * first call on it until the process ends.  Limit: ceil(N / 16) * 2 * C must
 * not exceed that size (e.g. N <= 21840 rows at C = 768, N <= 8192 at
 * C = 2048); larger shapes get GPT2_EINVAL with a message before anything is
 * launched, as do a NULL dw or db.  Every call on one GPU uses that GPU's same array and leaves its last
 * contents there (each partial row is written before it is read, so nothing
 * needs clearing); calls that overlap on one GPU (different streams, or other
 * threads) race on it and must be serialised by the caller.  Calls on one
 * stream are ordered and safe.  No device memory is allocated or freed. */
#define GPT2K_NOALLOC_SCRATCH_FLOATS ((size_t)1 << 21)
gpt2_status gpt2k_layernorm_backward_noalloc(float *dinp, float *dw, float *db, const float *dout, const float *inp,
                                             const float *w, const float *mean, const float *rstd, int N, int C,
                                             int accumulate, void *stream);

/* Calibration of the measurement (not a step of the training path): the
 * rates this device reaches, reported beside the vendor peaks.
 * gpt2k_probe_mfma launches one workgroup of 16 wavefronts per CU, each
 * running iters x 32 fp32 32x32x2 matrix instructions on register operands;
 * `out` is one device float (never written in practice), *flops (a HOST
 * double, may be NULL) receives the floating-point work launched; time the
 * call with events on `stream`.  gpt2k_probe_copy copies n floats
 * (n % 4 == 0, 16-byte aligned) with streaming loads and stores; a copy of
 * n floats moves 8n bytes.  GPT2_EINVAL for iters < 1 or a bad size. */
gpt2_status gpt2k_probe_mfma(float *out, int iters, double *flops, void *stream);
gpt2_status gpt2k_probe_copy(float *dst, const float *src, size_t n, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_MI_KERNELS_H */
