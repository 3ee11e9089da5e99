// Fused causal attention (fp32 MFMA, gfx950) over qkv rows [q | k | v] of
// width 3C, heads of hd = C / NH columns.  Supported for hd in {16, 32, 64}.
#pragma once
#include <hip/hip_runtime.h>

bool flash_attention_supported(int hd);

// Floats of workspace the calls below need: the forward's partial results of
// query blocks split between workgroups; for the backward the ds matrices and
// the dk/dv partials of key blocks split between workgroups.
size_t flash_attention_work(int B, int T, int C, int NH);

// out[B][T][C] = softmax(q k^T / sqrt(hd), causal) v per head;
// lse[B][NH][T] = log-sum-exp of each query's scaled scores.
hipError_t flash_attention_forward(float *out, float *lse, float *ws, const float *qkv, int B, int T, int C, int NH,
                                   hipStream_t s);

// Backward, first part: Dbuf[B][NH][T] = rowwise dout . out; dk and dv (the
// k and v blocks of dqkv, overwritten); and ds = p (dp - D) of every causal
// (t, u) into the workspace (flash_attention_ds), zero above the diagonal
// within each diagonal 128 x 128 tile.  The caller finishes with the
// product dq = ds K / sqrt(hd) (a causal GEMM that reads ds up to the end of
// each 128-row tile).
hipError_t flash_attention_backward_dkdv(float *dqkv, float *ws, float *Dbuf, const float *dout, const float *qkv,
                                         const float *out, const float *lse, int B, int T, int C, int NH,
                                         hipStream_t s);

// The [B][NH][T][T] ds matrices inside the workspace.
const float *flash_attention_ds(const float *ws);

// B*T*C floats of the workspace free once flash_attention_backward_dkdv has
// returned (its dk/dv partials are summed by then): room for the partial sums
// of the dq product.
float *flash_attention_dq_partial(float *ws, int B, int T, int NH);
