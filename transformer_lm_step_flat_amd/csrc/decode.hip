// Kernels of one decoding step (gfx950): each sequence's new position goes
// through every layer as a single row, the keys and values of the earlier
// positions being read from the rows the forward (or earlier steps) left in
// the qkv activations (the GeekNews page on the 3000-byte C GPT-2, "Cách KV
// caching hoạt động" and "Phép nhân ma trận nhanh": keep the cache, multiply
// only the new rows).  All of it is memory-bound (the weights are read once
// per step, the cache once per layer); at a few rows per step most launches
// are short enough that their fixed cost is a large part of their time.
#include "audit.h"
#include "common.h"
#include "decode.h"

namespace {

constexpr int RR = 4;  // rows of the row products per wave (grid.y covers the rest)
constexpr int NO = 4;  // outputs per wave
constexpr int JC = 4;  // float4s per lane per pass over K (a pass covers 1024 columns)

__device__ __forceinline__ float dot4(const floatx4 &a, const floatx4 &b) {
    return (a[0] * b[0] + a[1] * b[1]) + (a[2] * b[2] + a[3] * b[3]);
}

// out[r][o] = epi(xin[r] . W[o] + bias[o]) for the R rows (R small) and all
// OC outputs.  Each wave owns NO consecutive outputs and RR rows and keeps
// their dot products in registers: its lanes stride over K four floats at a
// time (16-byte loads; the weight matrix is read once per launch for each
// RR rows), and a wave reduction ends each dot product.  WS = 1: a workgroup
// is one wave doing all of K (K <= 1024).  WS = 4: the workgroup's four
// waves share the outputs and take a quarter of K each; their sums are added
// in wave order through LDS.  Every load a wave needs (weights, rows,
// LayerNorm gains, bias and residual) is issued before the arithmetic that
// waits on any of them.
// LN: xin = LayerNorm(x) with (lnw, lnb) over the K = C columns of each row,
// computed by each wave for its own rows (two passes, biased variance, eps
// 1e-5), so the LayerNorm needs no launch of its own.  epi: 0 store, 1 add
// aux[r][o] (residual; out may be aux), 2 GELU.  With pos_ptr, out is first
// moved by *pos_ptr rows of pos_stride floats (the position being decoded,
// read on the device).
template <int EPI, bool LN, int WS>
__global__ __launch_bounds__(64 * WS, 2) void rows_linear_kernel(float *out, long long ldo, const float *x, long long ldx,
                                                             const float *W, const float *bias, const float *aux,
                                                             long long ldaux, const float *lnw, const float *lnb, int R,
                                                             int K, int OC, const int *pos_ptr, long long pos_stride) {
    __shared__ float red[WS][NO * RR];
    if (pos_ptr) out += (long long)(*pos_ptr) * pos_stride;  // the decoded position's rows
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int o0 = blockIdx.x * NO, r0 = blockIdx.y * RR, nr = min(RR, R - r0);
    const int K4 = K >> 2, KS = (K4 + WS - 1) / WS;
    const int ks = wave * KS, ke = min(K4, ks + KS);
    const floatx4 *W4 = (const floatx4 *)W;
    const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
    // lane i < NO RR of wave 0 finishes output o0 + i / RR of row r0 + i % RR
    const int eo = o0 + lane / RR, er = lane % RR;
    const bool ep = wave == 0 && lane < NO * RR && eo < OC && er < nr;
    float eb = 0.0f, ea = 0.0f;
    if (ep) {
        if (bias) eb = bias[eo];
        if (EPI == 1) ea = aux[(long long)(r0 + er) * ldaux + eo];
    }
    floatx4 w[JC][NO], xv[JC][RR], g[JC], bb[JC];
    auto load = [&](int kb) {
#pragma unroll
        for (int j = 0; j < JC; j++) {
            const int k4 = kb + lane + 64 * j;
            const bool ok = k4 < ke;
#pragma unroll
            for (int c = 0; c < NO; c++) w[j][c] = ok && o0 + c < OC ? W4[(long long)(o0 + c) * K4 + k4] : z4;
#pragma unroll
            for (int r = 0; r < RR; r++)
                xv[j][r] = ok && r < nr ? *(const floatx4 *)(x + (long long)(r0 + r) * ldx + 4 * k4) : z4;
            if constexpr (LN) {
                g[j] = ok ? ((const floatx4 *)lnw)[k4] : z4;
                bb[j] = ok ? ((const floatx4 *)lnb)[k4] : z4;
            }
        }
    };
    load(ks);
    float mean[RR], rs[RR];
    if constexpr (LN) {
        // WS = 1: the registers hold the whole rows; WS = 4: each wave reads
        // the whole rows for the statistics (cache hits after the first)
        float s[RR], v[RR];
#pragma unroll
        for (int r = 0; r < RR; r++) s[r] = v[r] = 0.0f;
        if constexpr (WS == 1) {
#pragma unroll
            for (int j = 0; j < JC; j++)
#pragma unroll
                for (int r = 0; r < RR; r++) s[r] += (xv[j][r][0] + xv[j][r][1]) + (xv[j][r][2] + xv[j][r][3]);
        } else {
            for (int k4 = lane; k4 < K4; k4 += 64)
#pragma unroll
                for (int r = 0; r < RR; r++)
                    if (r < nr) {
                        const floatx4 t = *(const floatx4 *)(x + (long long)(r0 + r) * ldx + 4 * k4);
                        s[r] += (t[0] + t[1]) + (t[2] + t[3]);
                    }
        }
#pragma unroll
        for (int r = 0; r < RR; r++) mean[r] = wave_sum(s[r]) / K;
        if constexpr (WS == 1) {
#pragma unroll
            for (int j = 0; j < JC; j++)
                if (lane + 64 * j < K4)
#pragma unroll
                    for (int r = 0; r < RR; r++) {
                        const floatx4 d = xv[j][r] - mean[r];
                        v[r] += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
                    }
        } else {
            for (int k4 = lane; k4 < K4; k4 += 64)
#pragma unroll
                for (int r = 0; r < RR; r++)
                    if (r < nr) {
                        const floatx4 d = *(const floatx4 *)(x + (long long)(r0 + r) * ldx + 4 * k4) - mean[r];
                        v[r] += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
                    }
        }
#pragma unroll
        for (int r = 0; r < RR; r++) rs[r] = 1.0f / sqrtf(wave_sum(v[r]) / K + 1e-5f);
    }
    float acc[NO][RR];
#pragma unroll
    for (int c = 0; c < NO; c++)
#pragma unroll
        for (int r = 0; r < RR; r++) acc[c][r] = 0.0f;
    for (int kb = ks; kb < ke; kb += 64 * JC) {
        if (kb != ks) load(kb);
        if constexpr (LN) {
#pragma unroll
            for (int j = 0; j < JC; j++)
#pragma unroll
                for (int r = 0; r < RR; r++) xv[j][r] = (xv[j][r] - mean[r]) * rs[r] * g[j] + bb[j];
        }
        // columns past the end have zero weights, so their products vanish
#pragma unroll
        for (int j = 0; j < JC; j++)
#pragma unroll
            for (int r = 0; r < RR; r++)
#pragma unroll
                for (int c = 0; c < NO; c++) acc[c][r] += dot4(w[j][c], xv[j][r]);
    }
    float y = 0.0f;
#pragma unroll
    for (int c = 0; c < NO; c++)
#pragma unroll
        for (int r = 0; r < RR; r++) {
            const float t = wave_sum(acc[c][r]);
            if (lane == c * RR + r) y = t;
        }
    if constexpr (WS > 1) {
        if (lane < NO * RR) red[wave][lane] = y;
        __syncthreads();
        if (wave != 0 || lane >= NO * RR) return;
        y = red[0][lane];
#pragma unroll
        for (int q = 1; q < WS; q++) y += red[q][lane];
    }
    if (ep) {
        y += eb;
        if (EPI == 1) y += ea;
        if (EPI == 2) y = gelu_fwd(y);
        out[(long long)(r0 + er) * ldo + eo] = y;
    }
}

// Attention of the new query of (b, h) = blockIdx.x against the cached keys
// of one chunk of DKCH positions (blockIdx.y): scores, their max m, the
// exponentials' sum l and the weighted sum y of the chunk's values, written
// as a partial [y (hd) | m | l] at stride hd + 4 for the combine kernel.
// Thread t scores key t / 4 of the chunk over a quarter of the head dims;
// the value rows are loaded together with the keys.
constexpr int DKCH = 64;
constexpr int VPRE = 4;  // value rows per thread loaded ahead (all of them when hd <= 64)

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
    const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
    // thread (g, d4) sums keys g, g + ng, ... of the chunk at dims 4 d4 .. 4 d4 + 3
    const int ng = 256 / H4, g = tid / H4, d4 = tid % H4;
    floatx4 vr[VPRE];
#pragma unroll
    for (int i = 0; i < VPRE; i++) {
        const int j = g + ng * i;
        vr[i] = g < ng && j < n ? ((const floatx4 *)(rows + (long long)(u0 + j) * C3 + 2 * C))[d4] : z4;
    }
    {
        const int j = tid >> 2, qq = tid & 3;
        float s = 0.0f;
        if (j < n) {
            const floatx4 *k4 = (const floatx4 *)(rows + (long long)(u0 + j) * C3 + C);
            for (int d = qq; d < H4; d += 4) s += dot4(q4[d], k4[d]);
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
    floatx4 acc = z4;
    if (g < ng) {
#pragma unroll
        for (int i = 0; i < VPRE; i++) {
            const int j = g + ng * i;
            if (j < n) acc += sc[j] * vr[i];
        }
        for (int j = g + ng * VPRE; j < n; j += ng)
            acc += sc[j] * ((const floatx4 *)(rows + (long long)(u0 + j) * C3 + 2 * C))[d4];
    }
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
// partial slots per (b, h)).  The chunks' m and l are read once, all at a
// time, into LDS.
__global__ __launch_bounds__(64) void decode_attn_combine_kernel(float *atty, const float *ws, const int *pos_ptr,
                                                                 int nmax, int C, int NH) {
    __shared__ float sw[64];
    const int bh = blockIdx.x, b = bh / NH, h = bh % NH, hd = C / NH, lane = threadIdx.x;
    const int nchunk = *pos_ptr / DKCH + 1;  // <= nmax <= 16
    const float *p = ws + (long long)bh * nmax * (hd + 4);
    const float mc = lane < nchunk ? p[(long long)lane * (hd + 4) + hd] : -INFINITY;
    const float lc = lane < nchunk ? p[(long long)lane * (hd + 4) + hd + 1] : 0.0f;
    const float M = wave_max(mc);
    const float e = lane < nchunk ? __expf(mc - M) : 0.0f;
    sw[lane] = e;
    float L = 0.0f;
    for (int c = 0; c < nchunk; c++) L += __shfl(e, c) * __shfl(lc, c);
    __syncthreads();
    for (int d = lane; d < hd; d += 64) {
        float y = 0.0f;
        for (int c = 0; c < nchunk; c++) y += sw[c] * p[(long long)c * (hd + 4) + d];
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
    // max and its lowest index: each thread visits its indices in increasing
    // order (16-byte loads, four in flight, when the row is aligned), then
    // (value, index) pairs are reduced over the wavefront and the 16 waves
    float m = -INFINITY;
    int mi = V;
    int vs = 0;  // first index left to the scalar loop
    if (((uintptr_t)z & 15) == 0) {
        const int V4 = V / 4;
        const floatx4 *z4 = (const floatx4 *)z;
        for (int v4 = tid; v4 < V4; v4 += 4096) {
            floatx4 t[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int i = v4 + 1024 * u;
                t[u] = i < V4 ? z4[i] : (floatx4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            }
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    if (t[u][e] > m) {
                        m = t[u][e];
                        mi = 4 * (v4 + 1024 * u) + e;
                    }
        }
        vs = 4 * V4;
    }
    for (int v = vs + tid; v < V; v += 1024)
        if (z[v] > m) {
            m = z[v];
            mi = v;
        }
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(m, off);
        const int oi = __shfl_xor(mi, off);
        if (ov > m || (ov == m && oi < mi)) {
            m = ov;
            mi = oi;
        }
    }
    if ((tid & 63) == 0) {
        sv[tid >> 6] = m;
        si[tid >> 6] = mi;
    }
    __syncthreads();
    if (tid < 64) {
        m = tid < 16 ? sv[tid] : -INFINITY;
        mi = tid < 16 ? si[tid] : V;
        for (int off = 8; off > 0; off >>= 1) {
            const float ov = __shfl_xor(m, off);
            const int oi = __shfl_xor(mi, off);
            if (ov > m || (ov == m && oi < mi)) {
                m = ov;
                mi = oi;
            }
        }
        if (tid == 0) {
            best = mi < V ? mi : 0;  // a row with no finite maximum gives id 0
            sv[1023] = m;
        }
    }
    __syncthreads();
    const float zmax = sv[1023];
    const int amax = best;
    if (!coins) {
        if (tid == 0) next[b] = amax;
        return;
    }
    __syncthreads();  // every thread has read the maximum from sv[1023]
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
    if (ln && (!lnb || epi == 1 || ((uintptr_t)lnw & 15) || ((uintptr_t)lnb & 15))) return hipErrorInvalidValue;
    const bool split = K > 1024;  // four waves per output group, a quarter of K each
    if (AuditSink *au = audit_sink()) {
        const char *k = k_rows_linear_name(K);
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
    const dim3 grid((unsigned)((OC + NO - 1) / NO), (unsigned)((R + RR - 1) / RR));
#define RL_LAUNCH(E, L, WS)                                                                                        \
    hipLaunchKernelGGL((rows_linear_kernel<E, L, WS>), grid, dim3(64 * WS), 0, s, out, ldo, x, ldx, W, bias, aux, \
                       ldaux, lnw, lnb, R, K, OC, pos_ptr, pos_stride)
    if (split) {
        if (ln) {
            if (epi == 0) RL_LAUNCH(0, true, 4);
            else RL_LAUNCH(2, true, 4);
        } else {
            if (epi == 0) RL_LAUNCH(0, false, 4);
            else if (epi == 1) RL_LAUNCH(1, false, 4);
            else RL_LAUNCH(2, false, 4);
        }
    } else {
        if (ln) {
            if (epi == 0) RL_LAUNCH(0, true, 1);
            else RL_LAUNCH(2, true, 1);
        } else {
            if (epi == 0) RL_LAUNCH(0, false, 1);
            else if (epi == 1) RL_LAUNCH(1, false, 1);
            else RL_LAUNCH(2, false, 1);
        }
    }
#undef RL_LAUNCH
    return hipGetLastError();
}

const char *k_rows_linear_name(int K) { return K > 1024 ? "rows_linear_kernel<4>" : "rows_linear_kernel<1>"; }

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
