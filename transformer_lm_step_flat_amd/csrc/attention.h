// Fused causal attention (fp32 MFMA, gfx950) over qkv rows [q | k | v] of
// width 3C, heads of hd = C / NH columns.  Supported for hd in {16, 32, 64}.
#pragma once
#include <hip/hip_runtime.h>

bool flash_attention_supported(int hd);

// Floats of workspace the three calls below need (chunk partials of rows
// longer than one chunk).
size_t flash_attention_work(int B, int T, int C, int NH);

// out[B][T][C] = softmax(q k^T / sqrt(hd), causal) v per head;
// lse[B][NH][T] = log-sum-exp of each query's scaled scores.
hipError_t flash_attention_forward(float *out, float *lse, float *ws, const float *qkv, int B, int T, int C, int NH,
                                   hipStream_t s);

// Backward, in two calls: first dq (the q block of dqkv, overwritten) and
// Dbuf[B][NH][T] = rowwise dout . out; then dk and dv (the k and v blocks of
// dqkv, overwritten), which reads Dbuf.
hipError_t flash_attention_backward_dq(float *dqkv, float *Dbuf, float *ws, const float *dout, const float *qkv,
                                       const float *out, const float *lse, int B, int T, int C, int NH,
                                       hipStream_t s);
hipError_t flash_attention_backward_dkdv(float *dqkv, float *ws, const float *Dbuf, const float *dout,
                                         const float *qkv, const float *lse, int B, int T, int C, int NH,
                                         hipStream_t s);
