// Launchers of the decoding-step kernels (gfx950); each enqueues on `s` and
// returns hipGetLastError() (hipErrorInvalidValue for shapes it cannot take).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// out[r][o] = epi(xin[r] . W[o] + bias[o]) for r < R, o < OC; x rows ldx
// apart (K floats used), out rows ldo apart, W [OC][K] (out x in).  xin = x,
// or LayerNorm(x) with gains lnw and shifts lnb [K] when lnw is non-null.
// epi 0: store; 1: + aux[r][o] (aux rows ldaux apart; out may equal aux; not
// with LayerNorm); 2: GELU.  x, W, lnw and lnb 16-byte aligned, K and ldx
// multiples of 4.
// With pos_ptr (device int, may be NULL) out is first moved by *pos_ptr rows
// of pos_stride floats; pos_max bounds *pos_ptr (for the launch audit).
hipError_t k_rows_linear(float *out, long long ldo, const float *x, long long ldx, const float *W, const float *bias,
                         const float *aux, long long ldaux, const float *lnw, const float *lnb, int R, int K, int OC,
                         int epi, const int *pos_ptr, long long pos_stride, int pos_max, hipStream_t s);
const char *k_rows_linear_name(int K);  // the variant k_rows_linear runs for this K

// atty[b][:] = causal attention of query row (b, pos) over key/value rows
// (b, u <= pos) of qkv [B][T][3C] (q | k | v, heads of C / NH), pos =
// *pos_ptr read on the device; the keys are split into chunks whose partial
// results go through ws (decode_attention_work floats) and are merged in
// chunk order.
size_t decode_attention_work(int B, int T, int C, int NH);
hipError_t k_decode_attention(float *atty, float *ws, const float *qkv, const int *pos_ptr, int B, int T, int C,
                              int NH, hipStream_t s);

// *p = v (a launch, so that it can precede a replayed graph on the stream).
hipError_t k_set_int(int *p, int v, hipStream_t s);

// x[b][:] = wte[tokens[b]][:] + wpe[*pos_ptr][:]; ids outside [0, V) are read
// as the nearest valid one and set bit 1 of *err.  wpe has T rows.
hipError_t k_decode_embed(float *x, const int32_t *tokens, const float *wte, const float *wpe, const int *pos_ptr,
                          int32_t *err, int B, int C, int V, int T, hipStream_t s);

// next[b] from logits row b (ld floats apart, first V columns): argmax when
// coins is NULL, else the first v whose cumulative probability exceeds
// coins[b].
hipError_t k_sample(int32_t *next, const float *logits, long long ld, int B, int V, const float *coins,
                    const int *pos_ptr, long long pos_stride, int pos_max, hipStream_t s);
