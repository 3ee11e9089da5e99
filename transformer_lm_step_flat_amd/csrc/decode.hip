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

// out[r][o] = epi(x[r] . W[o] + bias[o]) for the R rows of x (R small) and
// all OC outputs.  A wavefront owns NCOL consecutive outputs; its lanes
// stride over K four floats at a time, reading each weight row once (the
// whole matrix once per launch), and the row sums are reduced across the
// wavefront.  epi: 0 store, 1 add aux[r][o] (residual; out may be aux),
// 2 GELU.
template <int NCOL, int EPI>
__global__ __launch_bounds__(256) void rows_linear_kernel(float *out, long long ldo, const float *x, long long ldx,
                                                          const float *W, const float *bias, const float *aux,
                                                          long long ldaux, int R, int K, int OC) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int o0 = (blockIdx.x * 4 + wave) * NCOL;
    const int r0 = blockIdx.y * RCH, nr = min(RCH, R - r0);
    if (o0 >= OC) return;  // the whole wavefront
    const int K4 = K / 4;
    const floatx4 *W4 = (const floatx4 *)W;
    float acc[NCOL][RCH];
#pragma unroll
    for (int c = 0; c < NCOL; c++)
#pragma unroll
        for (int r = 0; r < RCH; r++) acc[c][r] = 0.0f;
    for (int k4 = lane; k4 < K4; k4 += 64) {
        floatx4 w[NCOL];
#pragma unroll
        for (int c = 0; c < NCOL; c++)
            w[c] = o0 + c < OC ? W4[(long long)(o0 + c) * K4 + k4] : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RCH; r++) {
            if (r < nr) {
                const floatx4 xv = *(const floatx4 *)(x + (long long)(r0 + r) * ldx + 4 * k4);
#pragma unroll
                for (int c = 0; c < NCOL; c++)
                    acc[c][r] += (w[c][0] * xv[0] + w[c][1] * xv[1]) + (w[c][2] * xv[2] + w[c][3] * xv[3]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NCOL; c++)
#pragma unroll
        for (int r = 0; r < RCH; r++) {
            if (r < nr) {
                const float v = wave_sum(acc[c][r]);
                const int o = o0 + c;
                if (lane == 0 && o < OC) {
                    const long long rr = r0 + r;
                    float y = v + (bias ? bias[o] : 0.0f);
                    if (EPI == 1) y += aux[rr * ldaux + o];
                    if (EPI == 2) y = gelu_fwd(y);
                    out[rr * ldo + o] = y;
                }
            }
        }
}

// The new query of sequence b = blockIdx.x / NH, head h, against the cached
// keys u <= pos: p_u = softmax_u(q . k_u * scale), y = sum_u p_u v_u, written
// to atty[b][h hd ..].  One workgroup per (b, h); the scores stay in LDS.
__global__ __launch_bounds__(256) void decode_attention_kernel(float *atty, const float *qkv, int pos, int T, int C,
                                                               int NH, float scale) {
    __shared__ float p[1024];
    __shared__ floatx4 part[256];
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x / NH, h = blockIdx.x % NH, hd = C / NH, H4 = hd / 4;
    const long long C3 = 3LL * C;
    const float *rows = qkv + (long long)b * T * C3 + (long long)h * hd;  // q of position u at rows + u C3
    const floatx4 *q4 = (const floatx4 *)(rows + (long long)pos * C3);
    float mx = -INFINITY;
    for (int u = tid; u <= pos; u += 256) {
        const floatx4 *k4 = (const floatx4 *)(rows + (long long)u * C3 + C);
        float s = 0.0f;
        for (int d = 0; d < H4; d++) {
            const floatx4 a = q4[d], k = k4[d];
            s += (a[0] * k[0] + a[1] * k[1]) + (a[2] * k[2] + a[3] * k[3]);
        }
        s *= scale;
        p[u] = s;
        mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float sum = 0.0f;
    for (int u = tid; u <= pos; u += 256) {
        const float e = __expf(p[u] - mx);
        p[u] = e;
        sum += e;
    }
    sum = wave_sum(sum);
    __syncthreads();  // every wavefront has read the maxima
    if (lane == 0) red[wave] = sum;
    __syncthreads();  // the sums and every p[u] are visible
    sum = (red[0] + red[1]) + (red[2] + red[3]);
    // thread (g, d4): head dims 4 d4 .. 4 d4 + 3 of the keys u = g, g + ng, ...
    const int ng = 256 / H4, g = tid / H4, d4 = tid % H4;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (g < ng)
        for (int u = g; u <= pos; u += ng) acc += p[u] * ((const floatx4 *)(rows + (long long)u * C3 + 2 * C))[d4];
    part[tid] = acc;
    __syncthreads();
    if (tid < H4) {
        floatx4 t = part[tid];
        for (int k = 1; k < ng; k++) t += part[k * H4 + tid];
        *(floatx4 *)(atty + (long long)b * C + (long long)h * hd + 4 * tid) = t * (1.0f / sum);
    }
}

// The next token of row b = blockIdx.x of logits (first V columns): with
// coins == NULL the argmax (lowest index among equal maxima); otherwise the
// first v whose running sum of exp(z - max) exceeds coins[b] times the total
// (each thread sums a contiguous chunk; the chunk sums are scanned in a fixed
// order; the crossing chunk is walked again; V - 1 if rounding leaves no
// crossing).  One workgroup of 1024 threads per row.
__global__ __launch_bounds__(1024) void sample_kernel(int32_t *next, const float *logits, long long ld, int V,
                                                      const float *coins) {
    __shared__ float sv[1024];
    __shared__ int si[1024];
    __shared__ int best;
    const int b = blockIdx.x, tid = threadIdx.x;
    const float *z = logits + (long long)b * ld;
    const int chunk = (V + 1023) / 1024, c0 = min(tid * chunk, V), c1 = min(c0 + chunk, V);
    float m = -INFINITY;
    int mi = V;
    for (int v = c0; v < c1; v++)
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

}  // namespace

hipError_t k_rows_linear(float *out, long long ldo, const float *x, long long ldx, const float *W, const float *bias,
                         const float *aux, long long ldaux, int R, int K, int OC, int epi, hipStream_t s) {
    if (R <= 0 || K <= 0 || OC <= 0 || K % 4 || ldx % 4 || ((uintptr_t)x & 15) || ((uintptr_t)W & 15))
        return hipErrorInvalidValue;
    if (epi < 0 || epi > 2 || (epi == 1 && !aux)) return hipErrorInvalidValue;
    const bool wide = OC >= 8192;  // four outputs per wavefront where there are many
    const int ncol = wide ? 4 : 1;
    if (AuditSink *au = audit_sink()) {
        const char *k = wide ? "rows_linear_kernel<4>" : "rows_linear_kernel<1>";
        audit(au, k, "out", out, (long long)(R - 1) * ldo + OC, true);
        audit(au, k, "x", x, (long long)(R - 1) * ldx + K, false);
        audit(au, k, "W", W, (long long)OC * K, false);
        audit(au, k, "bias", bias, OC, false);
        if (epi == 1) audit(au, k, "aux", aux, (long long)(R - 1) * ldaux + OC, false);
        return hipSuccess;
    }
    dim3 grid((unsigned)((OC + 4 * ncol - 1) / (4 * ncol)), (unsigned)((R + RCH - 1) / RCH));
#define RL_LAUNCH(NC, E)                                                                                       \
    hipLaunchKernelGGL((rows_linear_kernel<NC, E>), grid, dim3(256), 0, s, out, ldo, x, ldx, W, bias, aux, ldaux, \
                       R, K, OC)
    if (wide) {
        if (epi == 0) RL_LAUNCH(4, 0);
        else if (epi == 1) RL_LAUNCH(4, 1);
        else RL_LAUNCH(4, 2);
    } else {
        if (epi == 0) RL_LAUNCH(1, 0);
        else if (epi == 1) RL_LAUNCH(1, 1);
        else RL_LAUNCH(1, 2);
    }
#undef RL_LAUNCH
    return hipGetLastError();
}

const char *k_rows_linear_name(int OC) { return OC >= 8192 ? "rows_linear_kernel<4>" : "rows_linear_kernel<1>"; }

hipError_t k_decode_attention(float *atty, const float *qkv, int pos, int B, int T, int C, int NH, hipStream_t s) {
    if (B <= 0 || NH <= 0 || C % NH || (C / NH) % 4 || C / NH > 1024 || T > 1024 || pos < 0 || pos >= T)
        return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        // rows b T + u, u <= pos, of each sequence's q | k | v
        const long long C3 = 3LL * C;
        audit(au, "decode_attention_kernel", "qkv", qkv, ((long long)(B - 1) * T + pos) * C3 + C3, false);
        audit(au, "decode_attention_kernel", "atty", atty, (long long)B * C, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(decode_attention_kernel, dim3((unsigned)(B * NH)), dim3(256), 0, s, atty, qkv, pos, T, C, NH,
                       1.0f / sqrtf((float)(C / NH)));
    return hipGetLastError();
}

hipError_t k_sample(int32_t *next, const float *logits, long long ld, int B, int V, const float *coins,
                    hipStream_t s) {
    if (B <= 0 || V <= 0 || ld < V) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        audit(au, "sample_kernel", "logits", logits, (long long)(B - 1) * ld + V, false);
        audit(au, "sample_kernel", "coins", coins, B, false);
        audit(au, "sample_kernel", "next", next, B, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(sample_kernel, dim3((unsigned)B), dim3(1024), 0, s, next, logits, ld, V, coins);
    return hipGetLastError();
}
