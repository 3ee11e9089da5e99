// Fused causal attention for gfx950 (fp32 MFMA), forward and backward,
// without materialising the T x T score or probability matrices.
//
// Definitions (GeekNews 3000-byte GPT-2 page, sections on the layers and the
// Transformer core: q.k products, the lower triangle, softmax, product with
// v): for one (batch, head), scale = 1/sqrt(hd),
//   s[t][u] = scale q_t . k_u  (u <= t),  p = softmax_u(s),  o_t = sum_u p[t][u] v_u.
// The forward keeps, per query, the running max and sum of the exponentials
// over key blocks (online softmax) and saves lse_t = max + log(sum).  The
// backward recomputes p from lse:
//   D_t = do_t . o_t,  dp[t][u] = do_t . v_u,  ds = p (dp - D_t),
//   dq_t = scale sum_u ds[t][u] k_u,  dk_u = scale sum_t ds[t][u] q_t,
//   dv_u = sum_t p[t][u] do_t.
//
// MFMA layout (v_mfma_f32_32x32x2_f32, lane l, half h = l / 32): the A
// operand is A[m = l % 32][k = slot h], B is B[k = slot h][n = l % 32], and
// the 32x32 result holds column l % 32, rows 8(r/4) + 4h + r%4 in register r.
// The forward and the dq kernel compute s^T = K Q^T so that a lane owns one
// query (a result column) and 32 keys (its rows): the softmax statistics are
// then per lane (plus its partner lane l ^ 32), and the probabilities sit
// exactly where o^T += V^T p^T needs them as its B operand.  The dk/dv kernel
// computes s = Q K^T so that a lane owns one key, and p / ds are in place as
// the A operand of dv += p^T dO and dk += ds^T Q.  Reductions over the head
// dimension use the k-split trick of the GEMM kernel: lane half h walks
// d = h*HD/2 + j.
//
// Every output element is written by exactly one lane, with sums in a fixed
// order: results are bitwise reproducible.
#include "attention.h"
#include "common.h"

namespace {

constexpr int QW = 32;     // queries (or keys) per wavefront
constexpr int NWAVE = 4;   // wavefronts per workgroup
constexpr int KB = 64;     // keys per block in the forward and dq kernels
constexpr int TB = 32;     // queries per block in the dk/dv kernel

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int r = 0; r < 16; r++) z[r] = 0.0f;
    return z;
}

__device__ __forceinline__ int row_of(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Load `rows` rows of HD floats (row stride `rs` floats, rows >= nvalid are
// zero) into registers: thread tid owns float4 number tid + 256*i.
template <int HD, int ROWS>
struct TileLoader {
    static constexpr int F4 = ROWS * HD / 4 / 256 > 0 ? ROWS * HD / 4 / 256 : 1;
    floatx4 r[F4];
    __device__ __forceinline__ void load(const float *base, long long rs, int row0, int nrows, int tid) {
#pragma unroll
        for (int i = 0; i < F4; i++) {
            int f = tid + 256 * i;
            int row = f / (HD / 4), c4 = f % (HD / 4);
            if (f < ROWS * HD / 4 && row0 + row < nrows)
                r[i] = *(const floatx4 *)(base + (long long)(row0 + row) * rs + 4 * c4);
            else
                r[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __device__ __forceinline__ void store(float *lds, int pitch, int tid) const {
#pragma unroll
        for (int i = 0; i < F4; i++) {
            int f = tid + 256 * i;
            if (f < ROWS * HD / 4) *(floatx4 *)&lds[(f / (HD / 4)) * pitch + 4 * (f % (HD / 4))] = r[i];
        }
    }
};

// s^T[mb] (keys 32mb.., this lane's query) = X[key][:] . frag   with X a [KB][pitch] LDS tile.
template <int HD>
__device__ __forceinline__ void keys_times_frag(floatx16 (&s)[2], const float *X, int pitch, const float *frag,
                                                int l32, int h) {
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
        s[mb] = zero16();
#pragma unroll
        for (int j4 = 0; j4 < HD / 8; j4++) {
            floatx4 a = *(const floatx4 *)&X[(32 * mb + l32) * pitch + h * (HD / 2) + 4 * j4];
#pragma unroll
            for (int e = 0; e < 4; e++)
                s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], frag[4 * j4 + e], s[mb], 0, 0, 0);
        }
    }
}

// HD = 16 has a single half-filled 32-row block for the head dimension.
template <int HD>
struct HeadBlocks {
    static constexpr int N = HD >= 32 ? HD / 32 : 1;
};

// acc^T[md] (head dims 32md.., this lane's query) += X^T P^T over the 64 keys
// of a block: X is a [KB][pitch] LDS tile, P (this lane's query, 32 keys per
// mb) is in registers.  For HD = 16 the head-dim block is half used: its
// other 16 rows get zero A values.
template <int HD>
__device__ __forceinline__ void accum_xt_pt_any(floatx16 (&acc)[HeadBlocks<HD>::N], const float *X, int pitch,
                                                const floatx16 (&p)[2], int l32, int h) {
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int u = 32 * mb + row_of(r, h);
#pragma unroll
            for (int md = 0; md < HeadBlocks<HD>::N; md++) {
                const int d = 32 * md + l32;
                const float a = d < HD ? X[u * pitch + d] : 0.0f;
                acc[md] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[mb][r], acc[md], 0, 0, 0);
            }
        }
}

// Write a per-wave transposed accumulator (lane: one query row t, registers:
// head dims) to global rows through LDS so that the stores are row-contiguous.
// Called by every wavefront of the workgroup (it contains a barrier); each
// wavefront uses its own LDS region.
template <int HD>
__device__ __forceinline__ void store_rows_t(float *dst, long long rs, int t0, int T, const floatx16 (&acc)[HeadBlocks<HD>::N],
                                             float mul, float *lds, int pitch, int lane) {
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int md = 0; md < HeadBlocks<HD>::N; md++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int d = 32 * md + row_of(r, h);
            if (d < HD) lds[l32 * pitch + d] = acc[md][r] * mul;
        }
    __syncthreads();
    // row-contiguous write-back: HD/4 float4 per row, 32 rows
    for (int f = lane; f < QW * HD / 4; f += 64) {
        const int row = f / (HD / 4), c4 = f % (HD / 4);
        if (t0 + row < T) *(floatx4 *)(dst + (long long)(t0 + row) * rs + 4 * c4) = *(const floatx4 *)&lds[row * pitch + 4 * c4];
    }
}

// ------------------------------------------------------------------ forward

template <int HD>
__global__ __launch_bounds__(256, 2) void flash_fwd_kernel(float *__restrict__ out, float *__restrict__ lse,
                                                           const float *__restrict__ qkv, int T, int C, int NH,
                                                           float scale) {
    constexpr int P = HD + 4;
    __shared__ __attribute__((aligned(16))) float Ks[KB * P];
    __shared__ __attribute__((aligned(16))) float Vs[KB * P];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int bh = blockIdx.y, b = bh / NH, hd_off = (bh % NH) * HD;
    const int nqb = (T + QW * NWAVE - 1) / (QW * NWAVE);
    const int q0 = (nqb - 1 - blockIdx.x) * QW * NWAVE;  // longest rows first
    const int tq0 = q0 + wave * QW, t = tq0 + l32;
    const long long rs = 3LL * C;
    const float *qb = qkv + (long long)b * T * rs + hd_off;

    float qf[HD / 2];
#pragma unroll
    for (int j4 = 0; j4 < HD / 8; j4++) {
        floatx4 v = t < T ? *(const floatx4 *)(qb + (long long)t * rs + h * (HD / 2) + 4 * j4) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; e++) qf[4 * j4 + e] = v[e] * scale;
    }
    floatx16 o[HeadBlocks<HD>::N];
#pragma unroll
    for (int md = 0; md < HeadBlocks<HD>::N; md++) o[md] = zero16();
    float m = -INFINITY, lsum = 0.0f;

    const int kend = min(T, q0 + QW * NWAVE);
    TileLoader<HD, KB> lk, lv;
    lk.load(qb + C, rs, 0, T, tid);
    lv.load(qb + 2 * C, rs, 0, T, tid);
    for (int k0 = 0; k0 < kend; k0 += KB) {
        __syncthreads();
        lk.store(Ks, P, tid);
        lv.store(Vs, P, tid);
        __syncthreads();
        if (k0 + KB < kend) {
            lk.load(qb + C, rs, k0 + KB, T, tid);
            lv.load(qb + 2 * C, rs, k0 + KB, T, tid);
        }
        if (k0 > tq0 + QW - 1) continue;  // every key of the block is after this wave's queries
        floatx16 s[2];
        keys_times_frag<HD>(s, Ks, P, qf, l32, h);
        float mx = m;
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int u = k0 + 32 * mb + row_of(r, h);
                const float v = (u > t || u >= T) ? -INFINITY : s[mb][r];
                s[mb][r] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
        const float alpha = __expf(m - mx);
        float ps = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float p = __expf(s[mb][r] - mx);
                s[mb][r] = p;
                ps += p;
            }
        ps += __shfl_xor(ps, 32, WAVE);
        lsum = lsum * alpha + ps;
        m = mx;
#pragma unroll
        for (int md = 0; md < HeadBlocks<HD>::N; md++) o[md] *= alpha;
        accum_xt_pt_any<HD>(o, Vs, P, s, l32, h);
    }
    __syncthreads();  // the K/V tiles become per-wave transpose space
    float *tr = (wave < 2 ? Ks : Vs) + (wave & 1) * QW * P;
    store_rows_t<HD>(out + (long long)b * T * C + hd_off, C, tq0, T, o, 1.0f / lsum, tr, P, lane);
    if (h == 0 && t < T) lse[(long long)bh * T + t] = m + __logf(lsum);
}

// ------------------------------------------------------------------ backward: dq and D

template <int HD>
__global__ __launch_bounds__(256, 2) void flash_bwd_dq_kernel(float *__restrict__ dqkv, float *__restrict__ Dbuf,
                                                              const float *__restrict__ dout,
                                                              const float *__restrict__ qkv,
                                                              const float *__restrict__ out,
                                                              const float *__restrict__ lse, int T, int C, int NH,
                                                              float scale) {
    constexpr int P = HD + 4;
    __shared__ __attribute__((aligned(16))) float Ks[KB * P];
    __shared__ __attribute__((aligned(16))) float Vs[KB * P];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int bh = blockIdx.y, b = bh / NH, hd_off = (bh % NH) * HD;
    const int nqb = (T + QW * NWAVE - 1) / (QW * NWAVE);
    const int q0 = (nqb - 1 - blockIdx.x) * QW * NWAVE;
    const int tq0 = q0 + wave * QW, t = tq0 + l32;
    const long long rs = 3LL * C;
    const float *qb = qkv + (long long)b * T * rs + hd_off;
    const float *dob = dout + (long long)b * T * C + hd_off;
    const float *ob = out + (long long)b * T * C + hd_off;

    float qf[HD / 2], dof[HD / 2];
    float dsum = 0.0f;
#pragma unroll
    for (int j4 = 0; j4 < HD / 8; j4++) {
        const bool ok = t < T;
        floatx4 q = ok ? *(const floatx4 *)(qb + (long long)t * rs + h * (HD / 2) + 4 * j4) : floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 d = ok ? *(const floatx4 *)(dob + (long long)t * C + h * (HD / 2) + 4 * j4) : floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 o = ok ? *(const floatx4 *)(ob + (long long)t * C + h * (HD / 2) + 4 * j4) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            qf[4 * j4 + e] = q[e] * scale;
            dof[4 * j4 + e] = d[e];
            dsum += d[e] * o[e];
        }
    }
    const float Dt = dsum + __shfl_xor(dsum, 32, WAVE);
    const float lt = t < T ? lse[(long long)bh * T + t] : 0.0f;
    if (h == 0 && t < T) Dbuf[(long long)bh * T + t] = Dt;

    floatx16 dq[HeadBlocks<HD>::N];
#pragma unroll
    for (int md = 0; md < HeadBlocks<HD>::N; md++) dq[md] = zero16();

    const int kend = min(T, q0 + QW * NWAVE);
    TileLoader<HD, KB> lk, lv;
    lk.load(qb + C, rs, 0, T, tid);
    lv.load(qb + 2 * C, rs, 0, T, tid);
    for (int k0 = 0; k0 < kend; k0 += KB) {
        __syncthreads();
        lk.store(Ks, P, tid);
        lv.store(Vs, P, tid);
        __syncthreads();
        if (k0 + KB < kend) {
            lk.load(qb + C, rs, k0 + KB, T, tid);
            lv.load(qb + 2 * C, rs, k0 + KB, T, tid);
        }
        if (k0 > tq0 + QW - 1) continue;
        floatx16 s[2], dp[2];
        keys_times_frag<HD>(s, Ks, P, qf, l32, h);
        keys_times_frag<HD>(dp, Vs, P, dof, l32, h);
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int u = k0 + 32 * mb + row_of(r, h);
                const float p = (u > t || u >= T) ? 0.0f : __expf(s[mb][r] - lt);
                s[mb][r] = p * (dp[mb][r] - Dt);  // ds
            }
        accum_xt_pt_any<HD>(dq, Ks, P, s, l32, h);
    }
    __syncthreads();
    float *tr = (wave < 2 ? Ks : Vs) + (wave & 1) * QW * P;
    store_rows_t<HD>(dqkv + (long long)b * T * rs + hd_off, rs, tq0, T, dq, scale, tr, P, lane);
}

// ------------------------------------------------------------------ backward: dk and dv

template <int HD>
__global__ __launch_bounds__(256, 2) void flash_bwd_dkdv_kernel(float *__restrict__ dqkv,
                                                                const float *__restrict__ dout,
                                                                const float *__restrict__ qkv,
                                                                const float *__restrict__ lse,
                                                                const float *__restrict__ Dbuf, int T, int C, int NH,
                                                                float scale) {
    constexpr int P = HD + 4;
    __shared__ __attribute__((aligned(16))) float Qs[TB * P];
    __shared__ __attribute__((aligned(16))) float Os[TB * P];  // dO tile
    __shared__ float Ls[TB], Ds[TB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int bh = blockIdx.y, b = bh / NH, hd_off = (bh % NH) * HD;
    const int u0w = blockIdx.x * QW * NWAVE;  // first key of the workgroup (earliest keys: most queries)
    const int u0 = u0w + wave * QW, u = u0 + l32;
    const long long rs = 3LL * C;
    const float *qb = qkv + (long long)b * T * rs + hd_off;
    const float *dob = dout + (long long)b * T * C + hd_off;

    float kf[HD / 2], vf[HD / 2];
#pragma unroll
    for (int j4 = 0; j4 < HD / 8; j4++) {
        const bool ok = u < T;
        floatx4 k = ok ? *(const floatx4 *)(qb + C + (long long)u * rs + h * (HD / 2) + 4 * j4) : floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 v = ok ? *(const floatx4 *)(qb + 2 * C + (long long)u * rs + h * (HD / 2) + 4 * j4) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            kf[4 * j4 + e] = k[e] * scale;
            vf[4 * j4 + e] = v[e];
        }
    }
    floatx16 dk[HeadBlocks<HD>::N], dv[HeadBlocks<HD>::N];
#pragma unroll
    for (int nd = 0; nd < HeadBlocks<HD>::N; nd++) dk[nd] = dv[nd] = zero16();

    TileLoader<HD, TB> lq, lo;
    const int tstart = u0w - u0w % TB;
    lq.load(qb, rs, tstart, T, tid);
    lo.load(dob, C, tstart, T, tid);
    for (int t0 = tstart; t0 < T; t0 += TB) {
        __syncthreads();
        lq.store(Qs, P, tid);
        lo.store(Os, P, tid);
        if (tid < TB) {
            Ls[tid] = t0 + tid < T ? lse[(long long)bh * T + t0 + tid] : 0.0f;
            Ds[tid] = t0 + tid < T ? Dbuf[(long long)bh * T + t0 + tid] : 0.0f;
        }
        __syncthreads();
        if (t0 + TB < T) {
            lq.load(qb, rs, t0 + TB, T, tid);
            lo.load(dob, C, t0 + TB, T, tid);
        }
        if (t0 + TB - 1 < u0) continue;  // every query of the block precedes this wave's keys
        // s[t][u] (rows: queries, column: this lane's key) and dp[t][u]
        floatx16 s = zero16(), dp = zero16();
#pragma unroll
        for (int j4 = 0; j4 < HD / 8; j4++) {
            floatx4 qa = *(const floatx4 *)&Qs[l32 * P + h * (HD / 2) + 4 * j4];
            floatx4 oa = *(const floatx4 *)&Os[l32 * P + h * (HD / 2) + 4 * j4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[e], kf[4 * j4 + e], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(oa[e], vf[4 * j4 + e], dp, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int tl = row_of(r, h), tt = t0 + tl;
            const float p = (tt < u || tt >= T || u >= T) ? 0.0f : __expf(s[r] - Ls[tl]);
            s[r] = p;                         // p
            dp[r] = p * (dp[r] - Ds[tl]);     // ds
        }
        // dv[u][d] += sum_t p[t][u] dO[t][d];  dk[u][d] += sum_t ds[t][u] q[t][d]
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int tl = row_of(r, h);
#pragma unroll
            for (int nd = 0; nd < HeadBlocks<HD>::N; nd++) {
                const int d = 32 * nd + l32;
                const float ob = d < HD ? Os[tl * P + d] : 0.0f;
                const float qv = d < HD ? Qs[tl * P + d] : 0.0f;
                dv[nd] = __builtin_amdgcn_mfma_f32_32x32x2f32(s[r], ob, dv[nd], 0, 0, 0);
                dk[nd] = __builtin_amdgcn_mfma_f32_32x32x2f32(dp[r], qv, dk[nd], 0, 0, 0);
            }
        }
    }
    // dk, dv: lane holds head dim 32nd + l32 of keys u0 + row_of(r, h): row-contiguous across lanes
    float *dkb = dqkv + (long long)b * T * rs + C + hd_off;
    float *dvb = dqkv + (long long)b * T * rs + 2 * C + hd_off;
#pragma unroll
    for (int nd = 0; nd < HeadBlocks<HD>::N; nd++) {
        const int d = 32 * nd + l32;
        if (d >= HD) continue;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int uu = u0 + row_of(r, h);
            if (uu < T) {
                dkb[(long long)uu * rs + d] = dk[nd][r] * scale;
                dvb[(long long)uu * rs + d] = dv[nd][r];
            }
        }
    }
}

template <int HD>
hipError_t launch_fwd(float *out, float *lse, const float *qkv, int B, int T, int C, int NH, hipStream_t s) {
    dim3 grid((T + QW * NWAVE - 1) / (QW * NWAVE), B * NH);
    hipLaunchKernelGGL(flash_fwd_kernel<HD>, grid, dim3(256), 0, s, out, lse, qkv, T, C, NH, 1.0f / sqrtf((float)HD));
    return hipGetLastError();
}

template <int HD>
hipError_t launch_bwd_dq(float *dqkv, float *Dbuf, const float *dout, const float *qkv, const float *out,
                         const float *lse, int B, int T, int C, int NH, hipStream_t s) {
    dim3 grid((T + QW * NWAVE - 1) / (QW * NWAVE), B * NH);
    hipLaunchKernelGGL(flash_bwd_dq_kernel<HD>, grid, dim3(256), 0, s, dqkv, Dbuf, dout, qkv, out, lse, T, C, NH,
                       1.0f / sqrtf((float)HD));
    return hipGetLastError();
}

template <int HD>
hipError_t launch_bwd_dkdv(float *dqkv, const float *Dbuf, const float *dout, const float *qkv, const float *lse,
                           int B, int T, int C, int NH, hipStream_t s) {
    dim3 grid((T + QW * NWAVE - 1) / (QW * NWAVE), B * NH);
    hipLaunchKernelGGL(flash_bwd_dkdv_kernel<HD>, grid, dim3(256), 0, s, dqkv, dout, qkv, lse, Dbuf, T, C, NH,
                       1.0f / sqrtf((float)HD));
    return hipGetLastError();
}

}  // namespace

bool flash_attention_supported(int hd) { return hd == 16 || hd == 32 || hd == 64; }

hipError_t flash_attention_forward(float *out, float *lse, const float *qkv, int B, int T, int C, int NH,
                                   hipStream_t s) {
    const int hd = C / NH;
    switch (hd) {
        case 16: return launch_fwd<16>(out, lse, qkv, B, T, C, NH, s);
        case 32: return launch_fwd<32>(out, lse, qkv, B, T, C, NH, s);
        case 64: return launch_fwd<64>(out, lse, qkv, B, T, C, NH, s);
    }
    return hipErrorInvalidValue;
}

hipError_t flash_attention_backward_dq(float *dqkv, float *Dbuf, const float *dout, const float *qkv,
                                       const float *out, const float *lse, int B, int T, int C, int NH,
                                       hipStream_t s) {
    switch (C / NH) {
        case 16: return launch_bwd_dq<16>(dqkv, Dbuf, dout, qkv, out, lse, B, T, C, NH, s);
        case 32: return launch_bwd_dq<32>(dqkv, Dbuf, dout, qkv, out, lse, B, T, C, NH, s);
        case 64: return launch_bwd_dq<64>(dqkv, Dbuf, dout, qkv, out, lse, B, T, C, NH, s);
    }
    return hipErrorInvalidValue;
}

hipError_t flash_attention_backward_dkdv(float *dqkv, const float *Dbuf, const float *dout, const float *qkv,
                                         const float *lse, int B, int T, int C, int NH, hipStream_t s) {
    switch (C / NH) {
        case 16: return launch_bwd_dkdv<16>(dqkv, Dbuf, dout, qkv, lse, B, T, C, NH, s);
        case 32: return launch_bwd_dkdv<32>(dqkv, Dbuf, dout, qkv, lse, B, T, C, NH, s);
        case 64: return launch_bwd_dkdv<64>(dqkv, Dbuf, dout, qkv, lse, B, T, C, NH, s);
    }
    return hipErrorInvalidValue;
}
