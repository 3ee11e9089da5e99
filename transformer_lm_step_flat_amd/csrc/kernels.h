// Launchers for the non-GEMM kernels of the training step (gfx950).
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

hipError_t k_fill(float *p, size_t n, float v, hipStream_t s);
hipError_t k_fill_i32(int32_t *p, size_t n, int32_t v, hipStream_t s);

// Validate ids (err |= 1 for an input, 2 for a target outside [0, V)) and
// sort the positions by (input id, position): order[rank] = position.  Below
// 8192 positions every position counts the keys below its own (O(BT^2)
// work, one launch); from there chunks of 1024 keys are sorted and each
// position's rank is found by binary search in every chunk (O(BT log BT)),
// with k_token_prep_work(BT) int32s of 8-byte-aligned workspace.
size_t k_token_prep_work(int BT);
hipError_t k_token_prep(const int32_t *inp, const int32_t *tgt, int32_t *order, int32_t *err, int32_t *work, int BT,
                        int V, hipStream_t s);
const char *k_token_prep_name(int BT);  // the kernel that gives the order

// out[b][t][:] = wte[inp[b][t]][:] + wpe[t][:]
hipError_t k_encoder_forward(float *out, const int32_t *inp, const float *wte, const float *wpe, int B, int T,
                             int C, int V, hipStream_t s);
// dwte[id][:] += sum of dout rows of that id (positions in ascending order);
// dwpe[t][:] += sum_b dout[b][t][:]
// part: B*T*C floats of workspace (segment sums).
hipError_t k_encoder_backward(float *dwte, float *dwpe, float *part, const float *dout, const int32_t *inp,
                              const int32_t *order, int B, int T, int C, int V, hipStream_t s);

hipError_t k_layernorm_forward(float *out, float *mean, float *rstd, const float *inp, const float *w,
                               const float *b, int N, int C, hipStream_t s);
// dinp (+)= LayerNorm input gradient; dw, db += weight/bias gradients, summed
// through `partial` ([ln_partials(N)][2C]) in a fixed order.
int ln_partials(int N);
hipError_t k_layernorm_backward(float *dinp, float *dw, float *db, float *partial, const float *dout,
                                const float *inp, const float *w, const float *mean, const float *rstd, int N,
                                int C, bool accumulate, hipStream_t s);
// With dw == NULL the row kernel only writes its partial rows [dw | db] (P x
// 2C floats at `partial`); k_ln_param_sums then adds the partials of all
// 2L + 1 LayerNorms of a backward pass (slot order: ln1 of each layer, ln2 of
// each layer, the final one; P x 2C floats per slot) into their gradients.
hipError_t k_ln_param_sums(float *w1, float *b1, float *w2, float *b2, float *w3, float *b3, int L,
                           const float *partial, int N, int C, hipStream_t s);

// dst[i] (+)= sum_{p < P} src[p * n + i]   (fixed order; n % 4 == 0, 16-byte aligned)
hipError_t k_sum_partials(float *dst, const float *src, int P, size_t n, bool accumulate, hipStream_t s);
// For L layers at once: dst1[l*n1 + i] += sum_p src1[(l*P + p)*n1 + i], and
// the same for region 2 (weight and bias gradients of one site of every layer).
hipError_t k_sum_layers(float *dst1, const float *src1, size_t n1, float *dst2, const float *src2, size_t n2, int P,
                       int L, hipStream_t s);
// Two such sums (regions of n1 and n2 floats, partial strides n1 and n2) in one launch.
hipError_t k_sum_partials2(float *dst1, const float *src1, size_t n1, float *dst2, const float *src2, size_t n2, int P,
                          bool accumulate, hipStream_t s);
// the same with partial rows ld apart
hipError_t k_sum_partials_ld(float *dst, const float *src, int P, size_t n, size_t ld, bool accumulate,
                             hipStream_t s);

// Causal row softmax in place over rows of T (T <= 1024): nrows = B*NH*T rows,
// row index t = row % T.  Writes zeros for t < u < round_up(t+1, CAUSAL_PAD).
hipError_t k_attn_softmax_forward(float *att, long long nrows, int T, hipStream_t s);
// dS = P * (dP - sum_u P dP), in place over dP; same zero padding.
hipError_t k_attn_softmax_backward(float *dp, const float *att, long long nrows, int T, hipStream_t s);

// Fused softmax cross-entropy over logits rows of width Vp (first V real):
// losses[r] = logsumexp - z[target]; logits <- (softmax - onehot) * dscale
// (0 in the padded columns).  If gate is non-null and *gate != 0 (an id of
// the batch was out of range), every row of the loss gradient is written as
// zeros and every loss as NaN instead, so that a backward over it adds
// nothing to the gradients.
hipError_t k_crossentropy(float *logits, float *losses, const int32_t *tgt, int BT, int V, int Vp, float dscale,
                          const int32_t *gate, hipStream_t s);
// Name of the kernel k_crossentropy launches for this padded vocabulary.
const char *k_crossentropy_name(int Vp);
// loss[0] = sum(losses) / n  (fixed order)
hipError_t k_mean(float *loss, const float *losses, int n, hipStream_t s);

// out = gelu(inp); dinp = dout * gelu'(inp)   (n % 4 == 0)
hipError_t k_gelu_forward(float *out, const float *inp, size_t n, hipStream_t s);
hipError_t k_gelu_backward(float *dinp, const float *inp, const float *dout, size_t n, hipStream_t s);

// AdamW over n floats; if gate is non-null and *gate != 0 nothing is read or
// written (the update of a batch with an out-of-range id is skipped).
hipError_t k_adamw(float *params, const float *grads, float *m, float *v, size_t n, float lr, float b1, float b2,
                   float eps, float wd, float c1, float c2, const int32_t *gate, hipStream_t s);
