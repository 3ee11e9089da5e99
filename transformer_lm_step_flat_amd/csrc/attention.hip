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
// The forward computes s^T = K Q^T so that a lane owns one query (a result
// column) and 32 keys (its rows): the softmax statistics are then per lane
// (plus its partner lane l ^ 32), and the probabilities sit exactly where
// o^T += V^T p^T needs them as its B operand.  The backward kernel computes
// s = Q K^T so that a lane owns one key, and p / ds are in place as the A
// operand of dv += p^T dO and dk += ds^T Q; it also stores ds (each
// wavefront's 32 x 32 block through a small LDS patch, as 16-byte row
// pieces), and dq = scale ds K is then a causal GEMM over the stored ds.
// Reductions over the head dimension use the k-split trick of the GEMM
// kernel: lane half h walks d = h*HD/2 + j.
//
// Every output element is written by exactly one lane, with sums in a fixed
// order: results are bitwise reproducible.
#include "attention.h"
#include "common.h"

namespace {

constexpr int QW = 32;     // queries (or keys) per wavefront
constexpr int NWAVE = 4;   // wavefronts per workgroup
constexpr int KB = 64;     // keys per block in the forward kernel
constexpr int TB = 32;     // queries per block in the dk/dv kernel

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int r = 0; r < 16; r++) z[r] = 0.0f;
    return z;
}

__device__ __forceinline__ int row_of(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Scores are kept in base 2: q (or k) is pre-multiplied by scale * log2(e),
// so that exp(scale q.k - lse) = 2^(s2 - lse * log2(e)) is one v_exp_f32.
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Load `rows` rows of HD floats (row stride `rs` floats, rows >= nvalid are
// zero) into registers: thread tid owns float4 number tid + 256*i.  The loads
// are issued unconditionally (a thread out of range reads row 0, which is
// always valid) and the zeroing is applied when the tile is stored, so that
// nothing waits for the loads until then: the next tile is in flight while
// the current one is consumed.
template <int HD, int ROWS>
struct TileLoader {
    static constexpr int F4 = ROWS * HD / 4 / 256 > 0 ? ROWS * HD / 4 / 256 : 1;
    floatx4 r[F4];
    bool ok[F4];
    __device__ __forceinline__ void load(const float *base, long long rs, int row0, int nrows, int tid) {
#pragma unroll
        for (int i = 0; i < F4; i++) {
            const int f = tid + 256 * i;
            const int row = f / (HD / 4), c4 = f % (HD / 4);
            ok[i] = f < ROWS * HD / 4 && row0 + row < nrows;
            r[i] = *(const floatx4 *)(base + (ok[i] ? (long long)(row0 + row) * rs + 4 * c4 : 0));
        }
    }
    __device__ __forceinline__ floatx4 value(int i) const {
        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
        return ok[i] ? r[i] : z;
    }
    __device__ __forceinline__ void store(float *lds, int pitch, int tid) const {
#pragma unroll
        for (int i = 0; i < F4; i++) {
            int f = tid + 256 * i;
            if (f < ROWS * HD / 4) *(floatx4 *)&lds[(f / (HD / 4)) * pitch + 4 * (f % (HD / 4))] = value(i);
        }
    }
    // The same tile transposed, [HD][pitch] (row index contiguous), so that
    // 4 consecutive rows of one column are one 16-byte LDS read.
    __device__ __forceinline__ void store_t(float *lds, int pitch, int tid) const {
#pragma unroll
        for (int i = 0; i < F4; i++) {
            int f = tid + 256 * i;
            if (f < ROWS * HD / 4) {
                const int row = f / (HD / 4), c = 4 * (f % (HD / 4));
                const floatx4 v = value(i);
#pragma unroll
                for (int e = 0; e < 4; e++) lds[(c + e) * pitch + row] = v[e];
            }
        }
    }
};

// s^T[mb] (keys 32mb.., this lane's query) = X[key][:] . frag   with X a [KB][pitch] LDS tile.
// The two 32-key halves are independent accumulation chains, interleaved.
template <int HD>
__device__ __forceinline__ void keys_times_frag(floatx16 (&s)[2], const float *X, int pitch, const float *frag,
                                                int l32, int h) {
    s[0] = zero16();
    s[1] = zero16();
#pragma unroll
    for (int j4 = 0; j4 < HD / 8; j4++) {
        floatx4 a0 = *(const floatx4 *)&X[l32 * pitch + h * (HD / 2) + 4 * j4];
        floatx4 a1 = *(const floatx4 *)&X[(32 + l32) * pitch + h * (HD / 2) + 4 * j4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[e], frag[4 * j4 + e], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[e], frag[4 * j4 + e], s[1], 0, 0, 0);
        }
    }
}

// HD = 16 has a single half-filled 32-row block for the head dimension.
template <int HD>
struct HeadBlocks {
    static constexpr int N = HD >= 32 ? HD / 32 : 1;
};

// acc^T[md] (head dims 32md.., this lane's query) += X^T P^T over the 64 keys
// of a block: Xt is the block's [HD][KB + 4] transposed LDS tile, P (this
// lane's query, 32 keys per mb) is in registers.  Register r of P holds key
// 8(r/4) + 4h + r%4, so the 4 registers 4g..4g+3 take 4 consecutive keys:
// one 16-byte read feeds 4 MFMAs.  For HD = 16 the head-dim block is half
// used: its other 16 rows get zero A values.
template <int HD>
__device__ __forceinline__ void accum_xt_pt_any(floatx16 (&acc)[HeadBlocks<HD>::N], const float *Xt,
                                                const floatx16 (&p)[2], int l32, int h) {
    constexpr int PT = KB + 4;
#pragma unroll
    for (int mb = 0; mb < 2; mb++)
#pragma unroll
        for (int g = 0; g < 4; g++)
#pragma unroll
            for (int md = 0; md < HeadBlocks<HD>::N; md++) {
                const int d = 32 * md + l32;
                const floatx4 a = d < HD ? *(const floatx4 *)&Xt[d * PT + 32 * mb + 8 * g + 4 * h]
                                         : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[md] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], p[mb][4 * g + i], acc[md], 0, 0, 0);
            }
}

// Write a per-wave transposed accumulator (lane: one row, registers: head
// dims) to `nrows` global rows (row stride rs) through LDS, so that the
// stores are row-contiguous.  Each lane's values are multiplied by its `mul`.
// Called by every wavefront of the workgroup (it contains a barrier); each
// wavefront passes its own LDS region of 32 x pitch floats.
template <int HD>
__device__ __forceinline__ void store_rows_t(float *dst, long long rs, int nrows,
                                             const floatx16 (&acc)[HeadBlocks<HD>::N], float mul, float *lds,
                                             int pitch, int lane) {
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int md = 0; md < HeadBlocks<HD>::N; md++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int d = 32 * md + row_of(r, h);
            if (d < HD) lds[l32 * pitch + d] = acc[md][r] * mul;
        }
    __syncthreads();
    for (int f = lane; f < QW * HD / 4; f += 64) {
        const int row = f / (HD / 4), c4 = f % (HD / 4);
        if (row < nrows) *(floatx4 *)(dst + (long long)row * rs + 4 * c4) = *(const floatx4 *)&lds[row * pitch + 4 * c4];
    }
}

// ------------------------------------------------------------------ work split (forward)
//
// Long causal rows are split so that no workgroup walks more than a few
// blocks in sequence: a forward workgroup takes 128 queries and one chunk of
// at most KCH of the keys they need.  A query block whose keys fit in one
// chunk writes its result directly; otherwise each chunk writes a partial
// (normalised output and log-sum-exp) to a workspace and a combine kernel
// merges the chunks in order.  (The dk/dv kernel splits its work differently;
// see there.)

constexpr int QBLK = QW * NWAVE;  // rows of a workgroup: 128
constexpr int KCH = 256;          // keys per chunk

__host__ __device__ inline int q_items(int qb, int T) {
    const int kend = min(T, (qb + 1) * QBLK);
    return (kend + KCH - 1) / KCH;
}
// chunks of query block qb that hold KCH keys (only the last can hold fewer)
__host__ __device__ inline int full_chunks(int qb, int T) { return min(T, (qb + 1) * QBLK) / KCH; }

// Work order: workgroup g of the one-dimensional grid takes first the full
// chunks of every (batch, head) in turn, then the shorter last chunks, so
// that the short ones fill the end of the launch.  Returns the (batch, head)
// index, the query block, the chunk and `first` = the item index of the
// block's chunk 0 (items numbered block by block within a (batch, head)).
__device__ __forceinline__ int decode_item(int g, int T, int &blk, int &chunk, int &first) {
    int nfull = 0, items = 0;
    for (int b = 0; b * QBLK < T; b++) {
        nfull += full_chunks(b, T);
        items += q_items(b, T);
    }
    const int npart = items - nfull, BH = gridDim.x / items;
    int bh, j;
    const bool full = g < BH * nfull;
    if (full) {
        bh = g / nfull;
        j = g % nfull;
    } else {
        bh = (g - BH * nfull) / npart;
        j = (g - BH * nfull) % npart;
    }
    first = 0;
    for (blk = 0;; blk++) {
        const int n = q_items(blk, T), f = full_chunks(blk, T);
        if (full) {
            if (j < f) { chunk = j; break; }
            j -= f;
        } else if (n > f) {
            if (j == 0) { chunk = n - 1; break; }
            j--;
        }
        first += n;
    }
    return bh;
}

// ------------------------------------------------------------------ forward

template <int HD>
__global__ __launch_bounds__(256, 3) void flash_fwd_kernel(float *__restrict__ out, float *__restrict__ lse,
                                                           float *__restrict__ ws, float *__restrict__ wlse,
                                                           const float *__restrict__ qkv, int T, int C, int NH,
                                                           int items, float scale) {
    constexpr int P = HD + 4;
    constexpr int PT = KB + 4;
    // K row-major [KB][P]; V transposed [HD][PT]; both reused as transpose space at the end
    constexpr int KS = KB * P, VS = (HD * PT > QW * NWAVE / 2 * P ? HD * PT : QW * NWAVE / 2 * P);
    __shared__ __attribute__((aligned(16))) float Ks[KS];
    __shared__ __attribute__((aligned(16))) float Vs[VS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
    int qb, chunk, first;
    const int bh = decode_item(blockIdx.x, T, qb, chunk, first);
    const int b = bh / NH, hd_off = (bh % NH) * HD;
    const int nch = q_items(qb, T);
    const int q0 = qb * QBLK;
    const int tq0 = q0 + wave * QW, t = tq0 + l32;
    const long long rs = 3LL * C;
    const float *qb_ptr = qkv + (long long)b * T * rs + hd_off;

    float qf[HD / 2];
#pragma unroll
    for (int j4 = 0; j4 < HD / 8; j4++) {
        floatx4 v = t < T ? *(const floatx4 *)(qb_ptr + (long long)t * rs + h * (HD / 2) + 4 * j4)
                          : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; e++) qf[4 * j4 + e] = v[e] * (scale * LOG2E);
    }
    floatx16 o[HeadBlocks<HD>::N];
#pragma unroll
    for (int md = 0; md < HeadBlocks<HD>::N; md++) o[md] = zero16();
    float m = -INFINITY, lsum = 0.0f;

    const int kc0 = chunk * KCH, kc1 = min(min(T, q0 + QBLK), kc0 + KCH);
    TileLoader<HD, KB> lk, lv;
    lk.load(qb_ptr + C, rs, kc0, T, tid);
    lv.load(qb_ptr + 2 * C, rs, kc0, T, tid);
    for (int k0 = kc0; k0 < kc1; k0 += KB) {
        __syncthreads();
        lk.store(Ks, P, tid);
        lv.store_t(Vs, PT, tid);
        __syncthreads();
        if (k0 + KB < kc1) {
            lk.load(qb_ptr + C, rs, k0 + KB, T, tid);
            lv.load(qb_ptr + 2 * C, rs, k0 + KB, T, tid);
        }
        if (k0 > tq0 + QW - 1) continue;  // every key of the block is after this wave's queries
        floatx16 s[2];
        keys_times_frag<HD>(s, Ks, P, qf, l32, h);
        float mx = m;
        if (k0 + KB - 1 > tq0 || k0 + KB > T) {  // the block crosses the diagonal or the end: mask
#pragma unroll
            for (int mb = 0; mb < 2; mb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int u = k0 + 32 * mb + row_of(r, h);
                    const float v = (u > t || u >= T) ? -INFINITY : s[mb][r];
                    s[mb][r] = v;
                    mx = fmaxf(mx, v);
                }
        } else {
#pragma unroll
            for (int mb = 0; mb < 2; mb++)
#pragma unroll
                for (int r = 0; r < 16; r++) mx = fmaxf(mx, s[mb][r]);
        }
        {
            const float2 hp = half_pair(mx);  // lanes i and i + 32 hold other keys of one query
            mx = fmaxf(hp.x, hp.y);
        }
        // a query that sees no key yet keeps m = -inf; exponentiate against 0 then
        const float mref = mx == -INFINITY ? 0.0f : mx;
        const float alpha = exp2_fast(m - mref);
        float ps = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float p = exp2_fast(s[mb][r] - mref);
                s[mb][r] = p;
                ps += p;
            }
        {
            const float2 hp = half_pair(ps);
            ps = hp.x + hp.y;
        }
        lsum = lsum * alpha + ps;
        m = mx;
#pragma unroll
        for (int md = 0; md < HeadBlocks<HD>::N; md++) o[md] *= alpha;
        accum_xt_pt_any<HD>(o, Vs, s, l32, h);
    }
    __syncthreads();  // the K/V tiles become per-wave transpose space
    float *tr = (wave < 2 ? Ks : Vs) + (wave & 1) * QW * P;
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    const float lse_t = lsum > 0.0f ? (m + __log2f(lsum)) * LN2 : -INFINITY;
    if (nch == 1) {
        store_rows_t<HD>(out + ((long long)b * T + tq0) * C + hd_off, C, T - tq0, o, inv, tr, P, lane);
        if (h == 0 && t < T) lse[(long long)bh * T + t] = lse_t;
    } else {
        const long long item = (long long)bh * items + first + chunk;
        store_rows_t<HD>(ws + (item * QBLK + wave * QW) * HD, HD, QW, o, inv, tr, P, lane);
        if (h == 0) wlse[item * QBLK + wave * QW + l32] = lse_t;
    }
}

// Merge the chunk partials of the forward: lse = log sum_c exp(lse_c);
// out = sum_c exp(lse_c - lse) out_c (chunks in order).  One thread per
// (row, 4 head dims) of the blocks that were split.
template <int HD>
__global__ __launch_bounds__(256) void flash_fwd_merge_kernel(float *__restrict__ out, float *__restrict__ lse,
                                                              const float *__restrict__ ws,
                                                              const float *__restrict__ wlse, int T, int C, int NH,
                                                              int BNH, int items) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int d4 = (int)(i % (HD / 4));
    const long long r = i / (HD / 4);
    const int t = (int)(r % T), bh = (int)(r / T);
    if (bh >= BNH) return;
    const int qb = t / QBLK, nch = q_items(qb, T);
    if (nch == 1) return;  // written directly by the forward kernel
    int first = 0;
    for (int q = 0; q < qb; q++) first += q_items(q, T);
    const long long base = (long long)bh * items + first;
    const int row = t % QBLK;
    float mx = -INFINITY;
    for (int c = 0; c < nch; c++) mx = fmaxf(mx, wlse[(base + c) * QBLK + row]);
    float ssum = 0.0f;
    for (int c = 0; c < nch; c++) ssum += __expf(wlse[(base + c) * QBLK + row] - mx);
    const float L = mx + __logf(ssum);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nch; c++) {
        const float w = __expf(wlse[(base + c) * QBLK + row] - L);
        acc += w * *(const floatx4 *)(ws + ((base + c) * QBLK + row) * HD + 4 * d4);
    }
    const int b = bh / NH, hd_off = (bh % NH) * HD;
    *(floatx4 *)(out + ((long long)b * T + t) * C + hd_off + 4 * d4) = acc;
    if (d4 == 0) lse[(long long)bh * T + t] = L;
}

// ------------------------------------------------------------------ backward: dk and dv
//
// Work split: the (batch, head, key block, query block) iterations are
// numbered key block by key block (128 keys, then its query blocks of TB
// from the block's diagonal on), (batch, head) after (batch, head), and the
// G workgroups (as many as can be resident) take equal contiguous ranges of
// them, so that all finish together.  A range is walked as segments, one per
// key block it touches.  A segment that covers all of its key block's query
// blocks writes dk and dv directly; otherwise it writes a partial sum to one
// of two slots of its workgroup (slot 0 for the segment that starts the
// range, slot 1 for the one that ends it), and flash_bwd_sum_kernel adds the
// partials of each split key block in workgroup order.

__host__ __device__ inline int kq_blocks(int kb, int T) { return (T - kb * QBLK + TB - 1) / TB; }
// first iteration of key block kb within a (batch, head)
__host__ __device__ inline int kq_start(int kb, int T) {
    int n = 0;
    for (int k = 0; k < kb; k++) n += kq_blocks(k, T);
    return n;
}
// range of workgroup g: [lo(g), lo(g + 1)) with lo(g) = g W / G
__host__ __device__ inline long long range_lo(long long g, long long W, long long G) { return g * W / G; }
// the workgroup whose range holds iteration i
__host__ __device__ inline long long range_of(long long i, long long W, long long G) { return ((i + 1) * G - 1) / W; }

// Logical workgroup of launch slot bid: workgroups are handed to the 8 XCDs
// round-robin, and each XCD gets one contiguous run of logical indices, so
// that neighbouring ranges (the same heads) share that XCD's L2.
__device__ __forceinline__ int xcd_run(int bid, int n) {
    const int X = 8;
    const int q = n / X, r = n % X;
    const int x = bid % X, loc = bid / X;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + loc;
}

template <int HD>
__global__ __launch_bounds__(256, 2) void flash_bwd_dkdv_kernel(float *__restrict__ dqkv, float *__restrict__ ws,
                                                                float *__restrict__ dsout,
                                                                const float *__restrict__ dout,
                                                                const float *__restrict__ qkv,
                                                                const float *__restrict__ lse,
                                                                const float *__restrict__ Dbuf, int T, int C, int NH,
                                                                int BH, float scale) {
    constexpr int P = HD + 4;
    // Q and dO tiles of TB queries, row-major, two buffers: the next block's
    // tiles are stored into the other buffer at the end of an iteration, so
    // one barrier per iteration suffices
    __shared__ __attribute__((aligned(16))) float Qs[2 * TB * P];
    __shared__ __attribute__((aligned(16))) float Os[2 * TB * P];
    __shared__ float Ls[2 * TB], Ds[2 * TB];
    // per wavefront, its 32 x 32 block of ds on the way to memory (row pitch PP)
    constexpr int PP = QW + 4;
    __shared__ __attribute__((aligned(16))) float Ps[NWAVE * QW * PP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int G = gridDim.x, g = xcd_run(blockIdx.x, G);
    const int nkb = (T + QBLK - 1) / QBLK, W1 = kq_start(nkb, T);
    const long long W = (long long)BH * W1;
    const long long lo_g = range_lo(g, W, G), hi_g = range_lo(g + 1, W, G);
    const long long rs = 3LL * C;
    TileLoader<HD, TB> lq, lo;
    // lse and D of a block's queries (threads tid < TB), loaded with its tiles
    float lse_next = 0.0f, d_next = 0.0f;
    bool ld_ok = false;
    auto load_rows = [&](int bh, int t0) {
        const int b = bh / NH, hd_off = (bh % NH) * HD;
        lq.load(qkv + (long long)b * T * rs + hd_off, rs, t0, T, tid);
        lo.load(dout + (long long)b * T * C + hd_off, C, t0, T, tid);
        ld_ok = tid < TB && t0 + tid < T;
        lse_next = lse[(long long)bh * T + (ld_ok ? t0 + tid : 0)];
        d_next = Dbuf[(long long)bh * T + (ld_ok ? t0 + tid : 0)];
    };
    auto store_rows = [&](int buf) {
        lq.store(Qs + buf * TB * P, P, tid);
        lo.store(Os + buf * TB * P, P, tid);
        if (tid < TB) {
            Ls[buf * TB + tid] = ld_ok ? lse_next * LOG2E : 0.0f;
            Ds[buf * TB + tid] = ld_ok ? d_next : 0.0f;
        }
    };
    // The segment that starts at iteration `it`: (batch, head), key block and
    // its query blocks [qfirst, qend).
    struct Seg {
        int bh, kb, qfirst, qend;
    };
    auto seg_at = [&](long long it) {
        Seg sg;
        sg.bh = (int)(it / W1);
        const int rem = (int)(it % W1);
        sg.kb = 0;
        while (sg.kb + 1 < nkb && kq_start(sg.kb + 1, T) <= rem) sg.kb++;
        sg.qfirst = rem - kq_start(sg.kb, T);
        sg.qend = (int)min((long long)kq_blocks(sg.kb, T), sg.qfirst + (hi_g - it));
        return sg;
    };
    // A segment's K and V rows (this lane's key, half the head dims per lane
    // half; a key past T reads row T - 1 and is zeroed when the segment
    // starts) and its first Q / dO tile are requested before the previous
    // segment's dk and dv are stored, so that their latency overlaps those stores.
    float kf[HD / 2], vf[HD / 2];
    auto request = [&](const Seg &sg) {
        const int b = sg.bh / NH, hd_off = (sg.bh % NH) * HD;
        const float *qb_ptr = qkv + (long long)b * T * rs + hd_off;
        const int uk = sg.kb * QBLK + wave * QW + l32, uc = uk < T ? uk : T - 1;
#pragma unroll
        for (int j4 = 0; j4 < HD / 8; j4++) {
            const floatx4 k = *(const floatx4 *)(qb_ptr + C + (long long)uc * rs + h * (HD / 2) + 4 * j4);
            const floatx4 v = *(const floatx4 *)(qb_ptr + 2 * C + (long long)uc * rs + h * (HD / 2) + 4 * j4);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                kf[4 * j4 + e] = k[e];
                vf[4 * j4 + e] = v[e];
            }
        }
        load_rows(sg.bh, sg.kb * QBLK + sg.qfirst * TB);
    };
    long long it = lo_g;
    Seg sg = seg_at(it);
    request(sg);
    for (;;) {
        const int bh = sg.bh, kb = sg.kb, qfirst = sg.qfirst, qend = sg.qend;
        const bool whole = qfirst == 0 && qend == kq_blocks(kb, T);
        const int slot = 2 * g + (it == lo_g ? 0 : 1);
        const int b = bh / NH, hd_off = (bh % NH) * HD;
        const int u0w = kb * QBLK;
        const int u0 = u0w + wave * QW, u = u0 + l32;
        // K pre-multiplied by scale log2(e); keys past T contribute nothing
#pragma unroll
        for (int i = 0; i < HD / 2; i++) {
            kf[i] = u < T ? kf[i] * (scale * LOG2E) : 0.0f;
            vf[i] = u < T ? vf[i] : 0.0f;
        }
        floatx16 dk[HeadBlocks<HD>::N], dv[HeadBlocks<HD>::N];
#pragma unroll
        for (int nd = 0; nd < HeadBlocks<HD>::N; nd++) dk[nd] = dv[nd] = zero16();

        const int tc0 = u0w + qfirst * TB, tc1 = min(T, u0w + qend * TB);
        // every wavefront is past the previous segment's last barrier: both buffers are free
        store_rows(0);
        __syncthreads();
        int cur = 0;
        for (int t0 = tc0; t0 < tc1; t0 += TB, cur ^= 1) {
            const bool more = t0 + TB < tc1;
            if (more) load_rows(bh, t0 + TB);
            const float *const Qc = Qs + cur * TB * P;
            const float *const Oc = Os + cur * TB * P;
            const float *const Lc = Ls + cur * TB;
            const float *const Dc = Ds + cur * TB;
            const bool edge = t0 + TB > T || u0 + QW > T;
            // This wave's 32 x 32 block of ds leaves as 16-byte stores: lane l takes
            // row l / 2, columns 8 i + 4 (l % 2) .. + 3 for i = 0..3 (one base address,
            // constant offsets).  T % 4 == 0 and u0 % 32 == 0, so a group of 4
            // columns lies wholly inside or outside [0, T).
            const int drow = lane >> 1, dcol = 4 * (lane & 1);
            float *const dsw = dsout + ((long long)bh * T + t0 + drow) * T + u0 + dcol;
            const bool row_ok = t0 + drow < T;
            if (t0 + TB - 1 < u0) {  // every query of the block precedes this wave's keys
                if (t0 < u0w + QBLK) {  // inside the diagonal 128 x 128 tile: ds = 0 for the dq product
                    // (a zero the compiler cannot see as a constant: it would keep a
                    // zero vector in registers through the whole loop otherwise)
                    float zf;
                    asm volatile("v_mov_b32 %0, 0" : "=v"(zf));
                    const floatx4 z = {zf, zf, zf, zf};
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (!edge || (row_ok && u0 + dcol + 8 * i < T)) *(floatx4 *)(dsw + 8 * i) = z;
                }
            } else {
            floatx16 s = zero16(), dp = zero16();
#pragma unroll
            for (int j4 = 0; j4 < HD / 8; j4++) {
                floatx4 qa = *(const floatx4 *)&Qc[l32 * P + h * (HD / 2) + 4 * j4];
                floatx4 oa = *(const floatx4 *)&Oc[l32 * P + h * (HD / 2) + 4 * j4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[e], kf[4 * j4 + e], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x2f32(oa[e], vf[4 * j4 + e], dp, 0, 0, 0);
                }
            }
            if (t0 < u0 + QW - 1 || edge) {  // crosses the diagonal or an end: mask
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int tl = row_of(r, h), tt = t0 + tl;
                    const float p = (tt < u || tt >= T || u >= T) ? 0.0f : exp2_fast(s[r] - Lc[tl]);
                    s[r] = p;                      // p
                    dp[r] = p * (dp[r] - Dc[tl]);  // ds
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int tl = row_of(r, h);
                    const float p = exp2_fast(s[r] - Lc[tl]);
                    s[r] = p;
                    dp[r] = p * (dp[r] - Dc[tl]);
                }
            }
            // ds[t][u] for the dq product goes through this wave's LDS patch (read
            // back as rows after the MFMAs below, when their operands are free).
            // The index is the lane's base plus a constant per register, so that
            // the constant becomes the instruction's offset.
            {
                const int pl = (wave * QW + 4 * h) * PP + l32;
#pragma unroll
                for (int r = 0; r < 16; r++) Ps[pl + (8 * (r >> 2) + (r & 3)) * PP] = dp[r];
            }
            // registers 4g..4g+3 hold queries 8g + 4h + 0..3; the B operands are
            // the rows of those queries at this lane's head dim: four 4-byte LDS
            // reads per 4 MFMAs (LDS reads issue beside the MFMAs of other
            // wavefronts, so no transposed copy of the tiles is kept)
            const int bq = 4 * h * P + l32;
#pragma unroll
            for (int g = 0; g < 4; g++)
#pragma unroll
                for (int nd = 0; nd < HeadBlocks<HD>::N; nd++) {
                    const int d = 32 * nd + l32;
                    floatx4 ob, qv;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        ob[i] = d < HD ? Oc[bq + (8 * g + i) * P + 32 * nd] : 0.0f;
                        qv[i] = d < HD ? Qc[bq + (8 * g + i) * P + 32 * nd] : 0.0f;
                    }
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        dv[nd] = __builtin_amdgcn_mfma_f32_32x32x2f32(s[4 * g + i], ob[i], dv[nd], 0, 0, 0);
                        dk[nd] = __builtin_amdgcn_mfma_f32_32x32x2f32(dp[4 * g + i], qv[i], dk[nd], 0, 0, 0);
                    }
                }
            {
                // the patch is this wavefront's alone: order its LDS writes before the reads
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const int pr = (wave * QW + drow) * PP + dcol;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const floatx4 v = *(const floatx4 *)&Ps[pr + 8 * i];
                    if (!edge || (row_ok && u0 + dcol + 8 * i < T)) *(floatx4 *)(dsw + 8 * i) = v;
                }
                // and the reads before the next iteration's writes
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            }  // keys after some queries of the block
            // the next block's tiles into the other buffer (last read in the
            // previous iteration, before its barrier), then one barrier
            if (more) store_rows(cur ^ 1);
            __syncthreads();
        }
        // the next segment's operands go out before this one's results
        const long long nxt = it + (qend - qfirst);
        if (nxt < hi_g) {
            sg = seg_at(nxt);
            request(sg);
        }
        // lane holds head dim 32nd + l32 of keys u0 + row_of(r, h): row-contiguous across lanes
        float *dkb, *dvb;
        long long krs;
        if (whole) {
            dkb = dqkv + (long long)b * T * rs + C + hd_off;
            dvb = dqkv + (long long)b * T * rs + 2 * C + hd_off;
            krs = rs;
        } else {
            dkb = ws + (long long)slot * 2 * QBLK * HD - (long long)u0w * HD;  // rows indexed by the key u
            dvb = dkb + QBLK * HD;
            krs = HD;
        }
#pragma unroll
        for (int nd = 0; nd < HeadBlocks<HD>::N; nd++) {
            const int d = 32 * nd + l32;
            if (d >= HD) continue;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int uu = u0 + row_of(r, h);
                if (uu < T) {
                    dkb[(long long)uu * krs + d] = dk[nd][r] * scale;
                    dvb[(long long)uu * krs + d] = dv[nd][r];
                }
            }
        }
        if (nxt >= hi_g) break;
        it = nxt;
    }  // segments
}

// D[bh][t] = dO_t . O_t over the head's HD dims, one thread per (b, t, head):
// consecutive threads take consecutive heads of a row.
template <int HD>
__global__ __launch_bounds__(256) void flash_bwd_D_kernel(float *__restrict__ Dbuf, const float *__restrict__ dout,
                                                          const float *__restrict__ out, int T, int C, int NH,
                                                          long long rows) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * NH) return;
    const long long bt = i / NH;
    const int hh = (int)(i % NH);
    const floatx4 *a = (const floatx4 *)(dout + bt * C + hh * HD);
    const floatx4 *o = (const floatx4 *)(out + bt * C + hh * HD);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < HD / 4; j++) {
        const floatx4 x = a[j], y = o[j];
        acc += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
    }
    const long long b = bt / T, t = bt % T;
    Dbuf[(b * NH + hh) * T + t] = acc;
}

// Sum the partials of dk and dv of the key blocks that were split between
// workgroups into dqkv, in workgroup order.  One thread per (key row, 4 head
// dims); rows of key blocks that one workgroup covered are left alone.
template <int HD>
__global__ __launch_bounds__(256) void flash_bwd_sum_kernel(float *__restrict__ dqkv, const float *__restrict__ ws,
                                                            int T, int C, int NH, int BH, int G) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int d4 = (int)(i % (HD / 4));
    const long long r = i / (HD / 4);
    const int t = (int)(r % T), bh = (int)(r / T);
    if (bh >= BH) return;
    const int kb = t / QBLK, nkb = (T + QBLK - 1) / QBLK;
    const long long W1 = kq_start(nkb, T), W = BH * W1;
    const long long S = bh * W1 + kq_start(kb, T), E = S + kq_blocks(kb, T);
    const long long ga = range_of(S, W, G), gb = range_of(E - 1, W, G);
    if (ga == gb) return;  // written directly
    const int row = t % QBLK;
    floatx4 ak = {0.f, 0.f, 0.f, 0.f}, av = {0.f, 0.f, 0.f, 0.f};
    for (long long g = ga; g <= gb; g++) {
        const long long slot = 2 * g + (range_lo(g, W, G) >= S ? 0 : 1);
        const float *p = ws + slot * 2 * QBLK * HD + (long long)row * HD + 4 * d4;
        ak += *(const floatx4 *)p;
        av += *(const floatx4 *)(p + QBLK * HD);
    }
    const long long rs = 3LL * C;
    const int b = bh / NH, hd_off = (bh % NH) * HD;
    *(floatx4 *)(dqkv + ((long long)b * T + t) * rs + C + hd_off + 4 * d4) = ak;
    *(floatx4 *)(dqkv + ((long long)b * T + t) * rs + 2 * C + hd_off + 4 * d4) = av;
}

// floats of the ds matrices at the start of the backward workspace (256-byte aligned)
size_t ds_floats(int B, int T, int NH) { return ((size_t)B * NH * T * T + 63) / 64 * 64; }

// forward items (query block chunks) of one (batch, head)
int total_items(int T) {
    int n = 0;
    for (int blk = 0; blk * QBLK < T; blk++) n += q_items(blk, T);
    return n;
}

template <int HD>
hipError_t launch_fwd(float *out, float *lse, float *ws, const float *qkv, int B, int T, int C, int NH,
                      hipStream_t s) {
    const int items = total_items(T);
    float *wlse = ws + (size_t)B * NH * items * QBLK * HD;
    hipLaunchKernelGGL(flash_fwd_kernel<HD>, dim3(items * B * NH), dim3(256), 0, s, out, lse, ws, wlse, qkv, T, C,
                       NH, items, 1.0f / sqrtf((float)HD));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || items == (T + QBLK - 1) / QBLK) return e;  // nothing was split
    const long long n = (long long)B * NH * T * (HD / 4);
    hipLaunchKernelGGL(flash_fwd_merge_kernel<HD>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, out, lse, ws,
                       wlse, T, C, NH, B * NH, items);
    return hipGetLastError();
}

// Workgroups of the dk/dv kernel: as many as are resident at once (256 CUs,
// two per CU by its register use), at most one per iteration.
int dkdv_groups(int B, int T, int NH, int hd) {
    const long long W = (long long)B * NH * kq_start((T + QBLK - 1) / QBLK, T);
    const long long cap = 256LL * 2;
    return (int)(W < cap ? W : cap);
}

template <int HD>
hipError_t launch_bwd_dkdv(float *dqkv, float *ws, float *Dbuf, const float *dout, const float *qkv,
                           const float *out, const float *lse, int B, int T, int C, int NH, hipStream_t s) {
    const long long rows = (long long)B * T;
    hipLaunchKernelGGL(flash_bwd_D_kernel<HD>, dim3((unsigned)((rows * NH + 255) / 256)), dim3(256), 0, s, Dbuf, dout,
                       out, T, C, NH, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = dkdv_groups(B, T, NH, HD);
    float *ds = ws, *kvws = ws + ds_floats(B, T, NH);
    hipLaunchKernelGGL(flash_bwd_dkdv_kernel<HD>, dim3(G), dim3(256), 0, s, dqkv, kvws, ds, dout, qkv, lse,
                       (const float *)Dbuf, T, C, NH, B * NH, 1.0f / sqrtf((float)HD));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long n = (long long)B * NH * T * (HD / 4);
    hipLaunchKernelGGL((flash_bwd_sum_kernel<HD>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dqkv,
                       (const float *)kvws, T, C, NH, B * NH, G);
    return hipGetLastError();
}

}  // namespace

bool flash_attention_supported(int hd) { return hd == 16 || hd == 32 || hd == 64; }

size_t flash_attention_work(int B, int T, int C, int NH) {
    const int hd = C / NH;
    const size_t fq = (size_t)B * NH * total_items(T) * QBLK * (hd + 1);
    // after ds: the dk/dv partials, later reused for the partial sums of dq
    const size_t kvp = (size_t)2 * dkdv_groups(B, T, NH, hd) * QBLK * 2 * hd, dqp = (size_t)B * T * C;
    const size_t kv = ds_floats(B, T, NH) + (kvp > dqp ? kvp : dqp);
    return fq > kv ? fq : kv;
}

const float *flash_attention_ds(const float *ws) { return ws; }

float *flash_attention_dq_partial(float *ws, int B, int T, int NH) { return ws + ds_floats(B, T, NH); }

hipError_t flash_attention_forward(float *out, float *lse, float *ws, const float *qkv, int B, int T, int C, int NH,
                                   hipStream_t s) {
    switch (C / NH) {
        case 16: return launch_fwd<16>(out, lse, ws, qkv, B, T, C, NH, s);
        case 32: return launch_fwd<32>(out, lse, ws, qkv, B, T, C, NH, s);
        case 64: return launch_fwd<64>(out, lse, ws, qkv, B, T, C, NH, s);
    }
    return hipErrorInvalidValue;
}

hipError_t flash_attention_backward_dkdv(float *dqkv, float *ws, float *Dbuf, const float *dout, const float *qkv,
                                         const float *out, const float *lse, int B, int T, int C, int NH,
                                         hipStream_t s) {
    switch (C / NH) {
        case 16: return launch_bwd_dkdv<16>(dqkv, ws, Dbuf, dout, qkv, out, lse, B, T, C, NH, s);
        case 32: return launch_bwd_dkdv<32>(dqkv, ws, Dbuf, dout, qkv, out, lse, B, T, C, NH, s);
        case 64: return launch_bwd_dkdv<64>(dqkv, ws, Dbuf, dout, qkv, out, lse, B, T, C, NH, s);
    }
    return hipErrorInvalidValue;
}
