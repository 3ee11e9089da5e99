// Kernels of one decoding step (gfx950): each sequence's new position goes
// through every layer as a single row, the keys and values of the earlier
// positions being read from the rows the forward (or earlier steps) left in
// the qkv activations (the GeekNews page on the 3000-byte C GPT-2, "Cách KV
// caching hoạt động" and "Phép nhân ma trận nhanh": keep the cache, multiply
// only the new rows).  All of it is bound by HBM: the weights are read once
// per step, the cache once per layer.
#include "audit.h"
#include "common.h"
#include "decode.h"

namespace {

constexpr int RCH = 8;  // rows per workgroup of the row products
constexpr int KPT = 2;  // float4s per thread of a LayerNorm-ed row (C <= 2048)

// Sum of v over the 256 threads of a workgroup for RCH values at once;
// red is [4][RCH] of LDS.  Fixed order: wavefront sums, then wave 0..3.
__device__ __forceinline__ void block_sums(float (&v)[RCH], float (*red)[RCH], int nr) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < RCH; r++)
        if (r < nr) {
            const float t = wave_sum(v[r]);
            if (lane == 0) red[wave][r] = t;
        }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RCH; r++) v[r] = (red[0][r] + red[1][r]) + (red[2][r] + red[3][r]);
    __syncthreads();
}

// out[r][o] = epi(xin[r] . W[o] + bias[o]) for the R rows (R small) and all
// OC outputs; a workgroup owns NC consecutive outputs and its 256 threads
// stride over K four floats at a time, so the whole weight matrix is read
// once per launch with 16-byte loads.  LN: xin = LayerNorm(x) with (lnw,
// lnb) over the K = C columns of each row, computed here (two passes over
// the row held in registers, biased variance, eps 1e-5), so the LayerNorm
// needs no launch of its own.  epi: 0 store, 1 add aux[r][o] (residual; out
// may be aux), 2 GELU.  With pos_ptr, out is first moved by *pos_ptr rows of
// pos_stride floats (the position being decoded, read on the device).
template <int NC, int EPI, bool LN>
__global__ __launch_bounds__(256) void rows_linear_kernel(float *out, long long ldo, const float *x, long long ldx,
                                                          const float *W, const float *bias, const float *aux,
                                                          long long ldaux, const float *lnw, const float *lnb, int R,
                                                          int K, int OC, const int *pos_ptr, long long pos_stride) {
    __shared__ float red[4][RCH];
    if (pos_ptr) out += (long long)(*pos_ptr) * pos_stride;  // the decoded position's rows
    __shared__ float acc_red[4][NC * RCH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int o0 = blockIdx.x * NC;
    const int r0 = blockIdx.y * RCH, nr = min(RCH, R - r0);
    const int K4 = K / 4;
    const floatx4 *W4 = (const floatx4 *)W;
    const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
    float acc[NC][RCH];
#pragma unroll
    for (int c = 0; c < NC; c++)
#pragma unroll
        for (int r = 0; r < RCH; r++) acc[c][r] = 0.0f;
    if constexpr (LN) {
        floatx4 xr[RCH][KPT];
        float sm[RCH];
#pragma unroll
        for (int r = 0; r < RCH; r++) {
            sm[r] = 0.0f;
#pragma unroll
            for (int j = 0; j < KPT; j++) {
                const int k4 = tid + 256 * j;
                xr[r][j] = (r < nr && k4 < K4) ? *(const floatx4 *)(x + (long long)(r0 + r) * ldx + 4 * k4) : z4;
                sm[r] += (xr[r][j][0] + xr[r][j][1]) + (xr[r][j][2] + xr[r][j][3]);
            }
        }
        block_sums(sm, red, nr);
        float mean[RCH], var[RCH];
#pragma unroll
        for (int r = 0; r < RCH; r++) {
            mean[r] = sm[r] / K;
            var[r] = 0.0f;
#pragma unroll
            for (int j = 0; j < KPT; j++)
                if (tid + 256 * j < K4) {
                    const floatx4 d = xr[r][j] - mean[r];
                    var[r] += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
                }
        }
        block_sums(var, red, nr);
#pragma unroll
        for (int j = 0; j < KPT; j++) {
            const int k4 = tid + 256 * j;
            if (k4 < K4) {
                const floatx4 g = ((const floatx4 *)lnw)[k4], bb = ((const floatx4 *)lnb)[k4];
                floatx4 w[NC];
#pragma unroll
                for (int c = 0; c < NC; c++) w[c] = o0 + c < OC ? W4[(long long)(o0 + c) * K4 + k4] : z4;
#pragma unroll
                for (int r = 0; r < RCH; r++) {
                    const float rs = 1.0f / sqrtf(var[r] / K + 1e-5f);
                    const floatx4 xv = (xr[r][j] - mean[r]) * rs * g + bb;
#pragma unroll
                    for (int c = 0; c < NC; c++)
                        acc[c][r] += (w[c][0] * xv[0] + w[c][1] * xv[1]) + (w[c][2] * xv[2] + w[c][3] * xv[3]);
                }
            }
        }
    } else {
        for (int k4 = tid; k4 < K4; k4 += 256) {
            floatx4 w[NC];
#pragma unroll
            for (int c = 0; c < NC; c++) w[c] = o0 + c < OC ? W4[(long long)(o0 + c) * K4 + k4] : z4;
#pragma unroll
            for (int r = 0; r < RCH; r++) {
                if (r < nr) {
                    const floatx4 xv = *(const floatx4 *)(x + (long long)(r0 + r) * ldx + 4 * k4);
#pragma unroll
                    for (int c = 0; c < NC; c++)
                        acc[c][r] += (w[c][0] * xv[0] + w[c][1] * xv[1]) + (w[c][2] * xv[2] + w[c][3] * xv[3]);
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NC; c++)
#pragma unroll
        for (int r = 0; r < RCH; r++)
            if (r < nr) {
                const float t = wave_sum(acc[c][r]);
                if (lane == 0) acc_red[wave][c * RCH + r] = t;
            }
    __syncthreads();
    if (tid < NC * RCH) {
        const int c = tid / RCH, r = tid % RCH, o = o0 + c;
        if (r < nr && o < OC) {
            const long long rr = r0 + r;
            float y = (acc_red[0][tid] + acc_red[1][tid]) + (acc_red[2][tid] + acc_red[3][tid]);
            y += bias ? bias[o] : 0.0f;
            if (EPI == 1) y += aux[rr * ldaux + o];
            if (EPI == 2) y = gelu_fwd(y);
            out[rr * ldo + o] = y;
        }
    }
}

// Attention of the new query of (b, h) = blockIdx.x against the cached keys
// of one chunk of DKCH positions (blockIdx.y): scores, their max m, the
// exponentials' sum l and the weighted sum y of the chunk's values, written
// as a partial [y (hd) | m | l] at stride hd + 4 for the combine kernel.
// Thread t works on key t / 4 of the chunk, a quarter of the head dims each.
constexpr int DKCH = 64;

__global__ __launch_bounds__(256) void decode_attn_partial_kernel(float *ws, const float *qkv, const int *pos_ptr, int T,
                                                                  int C, int NH, float scale) {
    __shared__ float sc[DKCH];
    __shared__ floatx4 part[256];
    __shared__ float ml[2];
    const int pos = *pos_ptr;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x, chunk = blockIdx.y, nchunk = gridDim.y;  // chunks of the whole T
    if (chunk * DKCH > pos) return;  // past the decoded position: no keys (the whole workgroup)
    const int b = bh / NH, h = bh % NH, hd = C / NH, H4 = hd / 4;
    const int u0 = chunk * DKCH, n = min(DKCH, pos + 1 - u0);
    const long long C3 = 3LL * C;
    const float *rows = qkv + (long long)b * T * C3 + (long long)h * hd;
    const floatx4 *q4 = (const floatx4 *)(rows + (long long)pos * C3);
    {
        const int j = tid >> 2, qq = tid & 3;
        float s = 0.0f;
        if (j < n) {
            const floatx4 *k4 = (const floatx4 *)(rows + (long long)(u0 + j) * C3 + C);
            for (int d = qq; d < H4; d += 4) {
                const floatx4 a = q4[d], k = k4[d];
                s += (a[0] * k[0] + a[1] * k[1]) + (a[2] * k[2] + a[3] * k[3]);
            }
        }
        s += dpp_move<0xB1>(s);  // the four quarters of the key's dot product
        s += dpp_move<0x4E>(s);
        if (qq == 0) sc[j] = j < n ? s * scale : -INFINITY;
    }
    __syncthreads();
    if (wave == 0) {
        const float v = sc[lane];
        const float m = wave_max(v);
        const float e = lane < n ? __expf(v - m) : 0.0f;
        const float l = wave_sum(e);
        sc[lane] = e;
        if (lane == 0) {
            ml[0] = m;
            ml[1] = l;
        }
    }
    __syncthreads();
    const int ng = 256 / H4, g = tid / H4, d4 = tid % H4;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (g < ng)
        for (int j = g; j < n; j += ng) acc += sc[j] * ((const floatx4 *)(rows + (long long)(u0 + j) * C3 + 2 * C))[d4];
    part[tid] = acc;
    __syncthreads();
    float *dst = ws + ((long long)bh * nchunk + chunk) * (hd + 4);
    if (tid < H4) {
        floatx4 t = part[tid];
        for (int k = 1; k < ng; k++) t += part[k * H4 + tid];
        *(floatx4 *)(dst + 4 * tid) = t;
    }
    if (tid == 0) {
        dst[hd] = ml[0];
        dst[hd + 1] = ml[1];
    }
}

// atty[b][h hd + d] = sum_c exp(m_c - M) y_c[d] / sum_c exp(m_c - M) l_c over
// the chunks c <= pos / DKCH of (b, h) = blockIdx.x, in chunk order (nmax
// partial slots per (b, h)).
__global__ __launch_bounds__(64) void decode_attn_combine_kernel(float *atty, const float *ws, const int *pos_ptr,
                                                                 int nmax, int C, int NH) {
    const int bh = blockIdx.x, b = bh / NH, h = bh % NH, hd = C / NH;
    const int nchunk = *pos_ptr / DKCH + 1;
    const float *p = ws + (long long)bh * nmax * (hd + 4);
    float M = -INFINITY;
    for (int c = 0; c < nchunk; c++) M = fmaxf(M, p[(long long)c * (hd + 4) + hd]);
    float L = 0.0f;
    for (int c = 0; c < nchunk; c++) L += __expf(p[(long long)c * (hd + 4) + hd] - M) * p[(long long)c * (hd + 4) + hd + 1];
    for (int d = threadIdx.x; d < hd; d += 64) {
        float y = 0.0f;
        for (int c = 0; c < nchunk; c++) y += __expf(p[(long long)c * (hd + 4) + hd] - M) * p[(long long)c * (hd + 4) + d];
        atty[(long long)b * C + (long long)h * hd + d] = y / L;
    }
}

// The next token of row b = blockIdx.x of logits (first V columns): with
// coins == NULL the argmax (lowest index among equal maxima); otherwise the
// first v whose running sum of exp(z - max) exceeds coins[b] times the total
// (each thread sums a contiguous chunk; the chunk sums are scanned in a fixed
// order; the crossing chunk is walked again; V - 1 if rounding leaves no
// crossing).  One workgroup of 1024 threads per row.
__global__ __launch_bounds__(1024) void sample_kernel(int32_t *next, const float *logits, long long ld, int V,
                                                      const float *coins, const int *pos_ptr, long long pos_stride) {
    if (pos_ptr) logits += (long long)(*pos_ptr) * pos_stride;
    __shared__ float sv[1024];
    __shared__ int si[1024];
    __shared__ int best;
    const int b = blockIdx.x, tid = threadIdx.x;
    const float *z = logits + (long long)b * ld;
    const int chunk = (V + 1023) / 1024, c0 = min(tid * chunk, V), c1 = min(c0 + chunk, V);
    // max and its lowest index: coalesced strided reads, then (value, index)
    // pairs reduced over the block
    float m = -INFINITY;
    int mi = V;
    for (int v = tid; v < V; v += 1024)
        if (z[v] > m) {
            m = z[v];
            mi = v;
        }
    sv[tid] = m;
    si[tid] = mi;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if (tid < s) {
            const int o = tid + s;
            if (sv[o] > sv[tid] || (sv[o] == sv[tid] && si[o] < si[tid])) {
                sv[tid] = sv[o];
                si[tid] = si[o];
            }
        }
        __syncthreads();
    }
    const float zmax = sv[0];
    const int amax = si[0];
    if (!coins) {
        if (tid == 0) next[b] = amax;
        return;
    }
    __syncthreads();  // every thread has read sv[0] and si[0]
    float cs = 0.0f;
    for (int v = c0; v < c1; v++) cs += __expf(z[v] - zmax);
    sv[tid] = cs;
    if (tid == 0) best = V;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan, fixed order
        const float t = tid >= off ? sv[tid - off] : 0.0f;
        __syncthreads();
        sv[tid] += t;
        __syncthreads();
    }
    const float excl = tid > 0 ? sv[tid - 1] : 0.0f;
    const float thr = coins[b] * sv[1023];
    if (c0 < c1 && excl <= thr) {
        float run = excl;
        for (int v = c0; v < c1; v++) {
            run += __expf(z[v] - zmax);
            if (run > thr) {
                atomicMin(&best, v);
                break;
            }
        }
    }
    __syncthreads();
    if (tid == 0) next[b] = best < V ? best : V - 1;
}

// x[b][:] = wte[id][:] + wpe[pos][:] for the token id of each sequence b at
// the decoded position pos = *pos_ptr; an id outside [0, V) is read as the
// nearest valid one and sets bit 1 of *err.  One workgroup per sequence.
__global__ __launch_bounds__(256) void decode_embed_kernel(float *x, const int32_t *tokens, const float *wte,
                                                           const float *wpe, const int *pos_ptr, int32_t *err, int C,
                                                           int V) {
    const int b = blockIdx.x, tid = threadIdx.x;
    const int raw = tokens[b], id = raw < 0 ? 0 : (raw >= V ? V - 1 : raw);
    if (tid == 0 && (raw < 0 || raw >= V)) atomicOr(err, 1);
    const floatx4 *we = (const floatx4 *)(wte + (long long)id * C);
    const floatx4 *pe = (const floatx4 *)(wpe + (long long)(*pos_ptr) * C);
    for (int c4 = tid; c4 < C / 4; c4 += 256) ((floatx4 *)(x + (long long)b * C))[c4] = we[c4] + pe[c4];
}

__global__ void set_int_kernel(int *p, int v) { *p = v; }

}  // namespace

hipError_t k_set_int(int *p, int v, hipStream_t s) {
    if (AuditSink *au = audit_sink()) {
        audit(au, "set_int_kernel", "p", p, 1, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(1), 0, s, p, v);
    return hipGetLastError();
}

hipError_t k_decode_embed(float *x, const int32_t *tokens, const float *wte, const float *wpe, const int *pos_ptr,
                          int32_t *err, int B, int C, int V, int T, hipStream_t s) {
    if (B <= 0 || C % 4 || V <= 0) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        audit(au, "decode_embed_kernel", "x", x, (long long)B * C, true);
        audit(au, "decode_embed_kernel", "tokens", tokens, B, false);
        audit(au, "decode_embed_kernel", "wte", wte, (long long)V * C, false);
        audit(au, "decode_embed_kernel", "wpe", wpe, (long long)T * C, false);  // rows pos < T
        audit(au, "decode_embed_kernel", "pos", pos_ptr, 1, false);
        audit(au, "decode_embed_kernel", "err", err, 1, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(decode_embed_kernel, dim3((unsigned)B), dim3(256), 0, s, x, tokens, wte, wpe, pos_ptr, err, C,
                       V);
    return hipGetLastError();
}

hipError_t k_rows_linear(float *out, long long ldo, const float *x, long long ldx, const float *W, const float *bias,
                         const float *aux, long long ldaux, const float *lnw, const float *lnb, int R, int K, int OC,
                         int epi, const int *pos_ptr, long long pos_stride, int pos_max, hipStream_t s) {
    if (R <= 0 || K <= 0 || OC <= 0 || K % 4 || ldx % 4 || ((uintptr_t)x & 15) || ((uintptr_t)W & 15))
        return hipErrorInvalidValue;
    if (epi < 0 || epi > 2 || (epi == 1 && !aux)) return hipErrorInvalidValue;
    const bool ln = lnw != nullptr;
    if (ln && (!lnb || K > 4 * 256 * KPT)) return hipErrorInvalidValue;
    const int nc = OC >= 2048 ? 4 : 2;
    if (AuditSink *au = audit_sink()) {
        const char *k = k_rows_linear_name(OC);
        // every position pos <= pos_max the launch may be replayed with
        audit(au, k, "out", out, (long long)(R - 1) * ldo + OC + (pos_ptr ? (long long)pos_max * pos_stride : 0), true);
        audit(au, k, "pos", pos_ptr, 1, false);
        audit(au, k, "x", x, (long long)(R - 1) * ldx + K, false);
        audit(au, k, "W", W, (long long)OC * K, false);
        audit(au, k, "bias", bias, OC, false);
        if (epi == 1) audit(au, k, "aux", aux, (long long)(R - 1) * ldaux + OC, false);
        audit(au, k, "lnw", lnw, ln ? K : 0, false);
        audit(au, k, "lnb", lnb, ln ? K : 0, false);
        return hipSuccess;
    }
    dim3 grid((unsigned)((OC + nc - 1) / nc), (unsigned)((R + RCH - 1) / RCH));
#define RL_LAUNCH(NC, E, L)                                                                                     \
    hipLaunchKernelGGL((rows_linear_kernel<NC, E, L>), grid, dim3(256), 0, s, out, ldo, x, ldx, W, bias, aux, ldaux, \
                       lnw, lnb, R, K, OC, pos_ptr, pos_stride)
    if (nc == 4) {
        if (ln) {
            if (epi == 0) RL_LAUNCH(4, 0, true);
            else if (epi == 2) RL_LAUNCH(4, 2, true);
            else return hipErrorInvalidValue;
        } else {
            if (epi == 0) RL_LAUNCH(4, 0, false);
            else if (epi == 1) RL_LAUNCH(4, 1, false);
            else RL_LAUNCH(4, 2, false);
        }
    } else {
        if (ln) {
            if (epi == 0) RL_LAUNCH(2, 0, true);
            else if (epi == 2) RL_LAUNCH(2, 2, true);
            else return hipErrorInvalidValue;
        } else {
            if (epi == 0) RL_LAUNCH(2, 0, false);
            else if (epi == 1) RL_LAUNCH(2, 1, false);
            else RL_LAUNCH(2, 2, false);
        }
    }
#undef RL_LAUNCH
    return hipGetLastError();
}

const char *k_rows_linear_name(int OC) { return OC >= 2048 ? "rows_linear_kernel<4>" : "rows_linear_kernel<2>"; }

size_t decode_attention_work(int B, int T, int C, int NH) {
    return (size_t)B * NH * ((T + DKCH - 1) / DKCH) * (C / NH + 4);
}

hipError_t k_decode_attention(float *atty, float *ws, const float *qkv, const int *pos_ptr, int B, int T, int C,
                              int NH, hipStream_t s) {
    if (B <= 0 || NH <= 0 || C % NH || (C / NH) % 4 || C / NH > 1024 || T > 1024 || T <= 0)
        return hipErrorInvalidValue;
    const int nmax = (T + DKCH - 1) / DKCH, hd = C / NH;
    if (AuditSink *au = audit_sink()) {
        // rows b T + u, u <= pos < T, of each sequence's q | k | v; nmax partial slots per (b, h)
        const long long C3 = 3LL * C, np = (long long)B * NH * nmax * (hd + 4);
        audit(au, "decode_attn_partial_kernel", "qkv", qkv, (long long)B * T * C3, false);
        audit(au, "decode_attn_partial_kernel", "pos", pos_ptr, 1, false);
        audit(au, "decode_attn_partial_kernel", "ws", ws, np, true);
        audit(au, "decode_attn_combine_kernel", "ws", ws, np, false);
        audit(au, "decode_attn_combine_kernel", "atty", atty, (long long)B * C, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(decode_attn_partial_kernel, dim3((unsigned)(B * NH), (unsigned)nmax), dim3(256), 0, s, ws, qkv,
                       pos_ptr, T, C, NH, 1.0f / sqrtf((float)hd));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_attn_combine_kernel, dim3((unsigned)(B * NH)), dim3(64), 0, s, atty, (const float *)ws,
                       pos_ptr, nmax, C, NH);
    return hipGetLastError();
}

hipError_t k_sample(int32_t *next, const float *logits, long long ld, int B, int V, const float *coins,
                    const int *pos_ptr, long long pos_stride, int pos_max, hipStream_t s) {
    if (B <= 0 || V <= 0 || ld < V) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        audit(au, "sample_kernel", "logits", logits,
              (long long)(B - 1) * ld + V + (pos_ptr ? (long long)pos_max * pos_stride : 0), false);
        audit(au, "sample_kernel", "pos", pos_ptr, 1, false);
        audit(au, "sample_kernel", "coins", coins, B, false);
        audit(au, "sample_kernel", "next", next, B, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(sample_kernel, dim3((unsigned)B), dim3(1024), 0, s, next, logits, ld, V, coins, pos_ptr,
                       pos_stride);
    return hipGetLastError();
}
