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
// o^T += V^T p^T needs them as its B operand (reductions over the head
// dimension use the k-split trick of the GEMM kernel: lane half h walks
// d = h*HD/2 + j).  The backward kernel uses v_mfma_f32_16x16x4_f32 and
// computes s = Q K^T so that a lane owns one key (a result column), and p /
// ds are in place as the A operand of dv += p^T dO and dk += ds^T Q; it also
// stores ds, and dq = scale ds K is then a causal GEMM over the stored ds.
//
// Every output element is written by exactly one lane, with sums in a fixed
// order: results are bitwise reproducible.
#include "audit.h"
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

// 16 bytes at byte offset voff + soff of base through a buffer resource of
// nbytes bytes: zeros past nbytes.  (A device function: a kernel body that
// names the buffer builtins fails the host compilation pass, which then
// drops the kernel's launch stub without a diagnostic.)
__device__ __forceinline__ floatx4 buf_load4(const float *base, int nbytes, unsigned voff, int soff) {
    const auto r = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, nbytes, 0x00020000);
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Load ROWS rows of HD floats (row stride rs floats) from row row0 into
// registers, rows at or past nrows as zeros: thread tid owns float4 number
// tid + 256 i, at row tid / (HD / 4) + i 256 / (HD / 4).  Buffer loads: one
// per-thread offset (the same for every tile), a scalar offset per load, no
// vector instructions for addresses.  The loads are issued at once and
// nothing waits for them until the tile is stored, so that the next tile is
// in flight while the current one is consumed.
template <int HD, int ROWS>
struct TileLoader {
    static constexpr int F4 = ROWS * HD / 4 / 256 > 0 ? ROWS * HD / 4 / 256 : 1;
    static constexpr int RPI = 256 / (HD / 4);  // rows per load index
    floatx4 r[F4];
    __device__ __forceinline__ void load(const float *base, long long rs, int row0, int nrows, int tid) {
        const unsigned voff = (unsigned)(4 * ((tid / (HD / 4)) * rs + 4 * (tid % (HD / 4))));
        const int nb = (int)(4 * (nrows - row0) * rs);
#pragma unroll
        for (int i = 0; i < F4; i++) r[i] = buf_load4(base + row0 * rs, nb, voff, (int)(4 * i * RPI * rs));
    }
    __device__ __forceinline__ void store(float *lds, int pitch, int tid) const {
#pragma unroll
        for (int i = 0; i < F4; i++) {
            const int f = tid + 256 * i;
            if (f < ROWS * HD / 4) *(floatx4 *)&lds[(f / (HD / 4)) * pitch + 4 * (f % (HD / 4))] = r[i];
        }
    }
};

// A 64-row tile that is stored transposed, [HD][pitch] (row index
// contiguous), so that 4 consecutive rows of one column are one 16-byte LDS
// read.  Thread tid loads row 16 wave + lane % 16, column groups 4 i +
// lane / 16 (i < HD / 16): the 64 lanes of one transposed store then write
// 16 rows of 4 columns, each of 32 banks twice (with 4 rows of 16 column
// groups per store, as in the row-major order, one bank takes 8 lanes).
// Rows at or past nrows read as zeros (buffer loads, as above).
template <int HD>
struct TileLoaderT {
    static constexpr int F4 = HD / 16;
    floatx4 r[F4];
    __device__ __forceinline__ void load(const float *base, long long rs, int row0, int nrows, int tid) {
        const int row = 16 * (tid >> 6) + (tid & 15), c0 = (tid >> 4) & 3;
        const unsigned voff = (unsigned)(4 * (row * rs + 4 * c0));
        const int nb = (int)(4 * (nrows - row0) * rs);
#pragma unroll
        for (int i = 0; i < F4; i++) r[i] = buf_load4(base + row0 * rs, nb, voff, 64 * i);
    }
    __device__ __forceinline__ void store_t(float *lds, int pitch, int tid) const {
        const int row = 16 * (tid >> 6) + (tid & 15), c0 = (tid >> 4) & 3;
#pragma unroll
        for (int i = 0; i < F4; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) lds[(4 * (4 * i + c0) + e) * pitch + row] = r[i][e];
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
    static_assert(KB == 64, "the transposed V tile has 64 rows");
    TileLoader<HD, KB> lk;
    TileLoaderT<HD> lv;
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
        // alpha is exactly 1 for a query whose running maximum did not move: when
        // that holds for the whole wavefront the rescaling of o is skipped (a
        // multiplication by 1 either way; the vector instructions it saves would
        // take issue cycles from the matrix unit)
        const bool moved = __ballot(mx != m) != 0;
        lsum = lsum * alpha + ps;
        m = mx;
        if (moved) {
#pragma unroll
            for (int md = 0; md < HeadBlocks<HD>::N; md++) o[md] *= alpha;
        }
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
// (row, 4 head dims) of the blocks that were split.  Up to MCH chunks (all of
// them for T <= MCH KCH) are loaded at once, more in a loop.
constexpr int MCH = 4;
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
    float L;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (nch <= MCH) {
        // every chunk's lse and partial row requested before the first use
        float l[MCH];
        floatx4 v[MCH];
#pragma unroll
        for (int c = 0; c < MCH; c++)
            if (c < nch) {
                l[c] = wlse[(base + c) * QBLK + row];
                v[c] = *(const floatx4 *)(ws + ((base + c) * QBLK + row) * HD + 4 * d4);
            }
        float mx = l[0];
#pragma unroll
        for (int c = 1; c < MCH; c++)
            if (c < nch) mx = fmaxf(mx, l[c]);
        float ssum = 0.0f;
#pragma unroll
        for (int c = 0; c < MCH; c++)
            if (c < nch) ssum += __expf(l[c] - mx);
        L = mx + __logf(ssum);
#pragma unroll
        for (int c = 0; c < MCH; c++)
            if (c < nch) acc += __expf(l[c] - L) * v[c];
    } else {
        float mx = -INFINITY;
        for (int c = 0; c < nch; c++) mx = fmaxf(mx, wlse[(base + c) * QBLK + row]);
        float ssum = 0.0f;
        for (int c = 0; c < nch; c++) ssum += __expf(wlse[(base + c) * QBLK + row] - mx);
        L = mx + __logf(ssum);
        for (int c = 0; c < nch; c++) {
            const float w = __expf(wlse[(base + c) * QBLK + row] - L);
            acc += w * *(const floatx4 *)(ws + ((base + c) * QBLK + row) * HD + 4 * d4);
        }
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

// The dk/dv kernel works with v_mfma_f32_16x16x4_f32 (A[i = l % 16][k = l / 16],
// B[k = l / 16][j = l % 16], result rows 4 (l / 16) + r, column l % 16 in
// register r): a wavefront owns KW = 16 keys (result columns of s = Q K^T),
// eight wavefronts the 128 keys of a key block, so that its persistent state
// (the keys' k and v rows and their dk, dv sums) is a quarter of what a 32-key
// wavefront holds and four wavefronts fit on each SIMD.  The Q and dO tiles
// go from memory straight into LDS (global_load_lds_dwordx4: lane L of a
// load writes the 16 bytes at the load's LDS base + 16 L), so that a tile in
// flight holds no registers.
constexpr int KW = 16;                // keys per wavefront
constexpr int NWB = QBLK / KW;        // wavefronts per workgroup: 8
constexpr int BWD_THREADS = 64 * NWB;  // 512

typedef __attribute__((address_space(3))) void lds_void;

// (the body is a device function: a kernel body that names the buffer
// builtins would fail the host compilation pass, which then drops the launch
// stub without a diagnostic)
template <int HD>
__device__ __forceinline__ void dkdv_body(float *__restrict__ dqkv, float *__restrict__ ws, float *__restrict__ dsout,
                                          const float *__restrict__ dout, const float *__restrict__ qkv,
                                          const float *__restrict__ lse, const float *__restrict__ Dbuf, int T, int C,
                                          int NH, int BH, float scale) {
    constexpr int KS = HD / 4;   // k steps of the s and dp products: lane group c takes head dims KS c ..
    constexpr int NB = HD / 16;  // 16-column blocks of dk and dv: column j of block nb is head dim NB j + nb
    constexpr int CH = HD / 4;        // 16-byte chunks per tile row
    constexpr int PC = CH + 1;        // chunks per LDS row: one of padding
    constexpr int P = 4 * PC;         // LDS row pitch in floats
    constexpr int NI = (TB * PC + 63) / 64;  // 64-lane loads per tile
    constexpr int TS = 64 * NI * 4;   // floats per tile buffer (the last load's tail is slack)
    // Q and dO tiles of TB queries (rows of HD floats, P apart, so that the
    // reads below meet every bank evenly) and [lse of the TB queries | their
    // D], two buffers: the next block's tiles are loaded into one while the
    // other is read, and one barrier per block suffices.  The key block's k
    // rows (QBLK rows, P apart) follow.  One array: every LDS read is a
    // per-lane base plus a constant offset.
    constexpr int NKI = (QBLK * PC + 63) / 64;  // 64-lane loads of the k rows
    constexpr int KT = 64 * NKI * 4;
    // buffer b: Q at 2 TS b, dO at 2 TS b + TS, [lse | D] at 4 TS + 2 TB b; the
    // k rows at 4 TS + 4 TB
    __shared__ __attribute__((aligned(16))) float sm[4 * TS + 4 * TB + KT];
    float *const Kt = sm + 4 * TS + 4 * TB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane >> 4, j = lane & 15;
    const int G = gridDim.x, g = xcd_run(blockIdx.x, G);
    const int nkb = (T + QBLK - 1) / QBLK, W1 = kq_start(nkb, T);
    const long long W = (long long)BH * W1;
    const long long lo_g = range_lo(g, W, G), hi_g = range_lo(g + 1, W, G);
    const long long rs = 3LL * C;
    const int Tp = (T + 3) & ~3;  // ds row pitch
    // Loads of the tiles of the block of queries t0 .. t0 + TB - 1 into buffer
    // buf, as buffer loads straight into LDS: load I of a tile fills chunk
    // positions 64 I .. 64 I + 63 of its buffer (row p / PC, chunk p % PC; a
    // padding chunk or a position past the tile reads a chunk of the tile's
    // rows and is never read back).  Wavefront w makes load w of the Q and of
    // the dO tile (wavefront 0 also the loads from NWB on), the last
    // wavefront the lse and D values.  The resources start at row t0 and end
    // at row T: rows past T read as zeros.  A lane's offset within a load is
    // the same for every block: computed once.
    auto lane_off = [&](int inst, long long stride) {
        const int p = 64 * inst + lane, t = min(p / PC, TB - 1), k = min(p % PC, CH - 1);
        return (unsigned)(4 * (t * stride + 4 * k));
    };
    const unsigned offq = lane_off(wave, rs), offo = lane_off(wave, C);
    auto issue = [&](int buf, int bh, int t0) {
        float *const Qd = sm + 2 * TS * buf, *const Od = Qd + TS, *const Ld = sm + 4 * TS + 2 * TB * buf;
        const int b = bh / NH, hd_off = (bh % NH) * HD;
        const auto qr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(qkv + ((long long)b * T + t0) * rs + hd_off), (short)0, (int)(4 * (T - t0) * rs), 0x00020000);
        const auto orr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(dout + ((long long)b * T + t0) * C + hd_off), (short)0, 4 * (T - t0) * C, 0x00020000);
        if (wave < NI) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void *)(Qd + 256 * wave), 16, offq, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(orr, (lds_void *)(Od + 256 * wave), 16, offo, 0, 0, 0);
        }
        if (wave == 0) {
            for (int I = NWB; I < NI; I++) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void *)(Qd + 256 * I), 16, lane_off(I, rs), 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(orr, (lds_void *)(Od + 256 * I), 16, lane_off(I, C), 0, 0, 0);
            }
        }
        if (wave == NWB - 1) {
            const auto lr = __builtin_amdgcn_make_buffer_rsrc((void *)(lse + (long long)bh * T + t0), (short)0,
                                                              4 * (T - t0), 0x00020000);
            const auto dr = __builtin_amdgcn_make_buffer_rsrc((void *)(Dbuf + (long long)bh * T + t0), (short)0,
                                                              4 * (T - t0), 0x00020000);
            if (lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(lr, (lds_void *)Ld, 4, 4 * lane, 0, 0, 0);
            else __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void *)Ld, 4, 4 * (lane - 32), 0, 0, 0);
        }
    };
    // this wavefront's tile loads have landed (other wavefronts': after the barrier that follows)
    auto loads_done = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
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
    // A segment's k and v rows (this lane's key j, head dims KS c ..; a key
    // past T reads row T - 1 and is zeroed when the segment starts) and its
    // first Q / dO tiles (into buffer 0) are requested before the previous
    // segment's dk and dv are stored, so that their latency overlaps those stores.
    // (the k rows go to LDS, the v rows to registers: both in registers would
    // not leave room for four wavefronts per SIMD)
    float vf[KS];
    auto request = [&](const Seg &sg) {
        const int b = sg.bh / NH, hd_off = (sg.bh % NH) * HD;
        const float *qb_ptr = qkv + (long long)b * T * rs + hd_off;
        const int uk = sg.kb * QBLK + wave * KW + j, uc = uk < T ? uk : T - 1;
#pragma unroll
        for (int m = 0; m < KS / 4; m++) {
            const floatx4 v = *(const floatx4 *)(qb_ptr + 2 * C + (long long)uc * rs + KS * c + 4 * m);
#pragma unroll
            for (int e = 0; e < 4; e++) vf[4 * m + e] = v[e];
        }
        // the key block's k rows: row p / PC, chunk p % PC of position p (a padding
        // chunk reads a valid chunk; a row past T reads row T - 1: its scores are masked)
        const char *const kbase = (const char *)(qb_ptr + C);
        int ln = lane;
        asm volatile("" : "+v"(ln));
        for (int I = wave; I < NKI; I += NWB) {
            const int p = 64 * I + ln, t = p / PC, k = min(p % PC, CH - 1);
            const unsigned off = (unsigned)(min(sg.kb * QBLK + t, T - 1) * (int)rs + 4 * k) * 4u;
            __builtin_amdgcn_global_load_lds(kbase + off, (lds_void *)(Kt + 256 * I), 16, 0, 0);
        }
        issue(0, sg.bh, sg.kb * QBLK + sg.qfirst * TB);
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
        const int u0 = u0w + wave * KW, u = u0 + j;
        // keys past T contribute nothing
#pragma unroll
        for (int i = 0; i < KS; i++) vf[i] = u < T ? vf[i] : 0.0f;
        const float sl2e = scale * LOG2E;  // scores in base 2
        floatx4 dk[NB], dv[NB];
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int r = 0; r < 4; r++) dk[nb][r] = dv[nb][r] = 0.0f;

        const int tc0 = u0w + qfirst * TB, tc1 = min(T, u0w + qend * TB);
        // ds[t][u] of register r of half qh: query t0 + 16 qh + 4 c + r, key u,
        // written with buffer stores into the head's ds matrix (a resource that
        // ends at row T: rows past T are dropped; T Tp < 2^29).  Rows are Tp
        // floats apart; columns T .. Tp - 1 take the zeros of the keys past T,
        // and nothing is written at or past column Tp.
        const auto dsr = __builtin_amdgcn_make_buffer_rsrc((void *)(dsout + (long long)bh * T * Tp), (short)0,
                                                           4 * T * Tp, 0x00020000);
        const bool col_ok = u < Tp;
        auto ds_store = [&](float v, unsigned voff, int row) {
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), dsr, voff, 4 * row * Tp, 0);
        };
        // the segment's first tiles (buffer 0) were requested with its k and v rows
        loads_done();
        __syncthreads();
        // blocks of TB queries, each from buffer cur (its tiles were requested
        // before); the next block's tiles go into the other buffer meanwhile
        int cur = 0;
        for (int t0 = tc0; t0 < tc1; t0 += TB, cur ^= 1) {
            const float *const Qc = sm + 2 * TS * cur, *const Oc = Qc + TS, *const Lc = sm + 4 * TS + 2 * TB * cur;
            if (t0 + TB < tc1) issue(cur ^ 1, bh, t0 + TB);
            const bool edge = t0 + TB > T || u0 + KW > T;
            // the lane's byte offset of row t0 + 4 c, column u (rows 16 qh + r further
            // on are the stores' scalar offsets)
            const unsigned dso = (unsigned)(4 * ((t0 + 4 * c) * Tp + u));
            if (t0 + TB - 1 < u0) {  // every query of the block precedes this wave's keys
                if (t0 < u0w + QBLK && col_ok) {  // inside the diagonal 128 x 128 tile: ds = 0 for the dq product
#pragma unroll
                    for (int qh = 0; qh < 2; qh++)
#pragma unroll
                        for (int r = 0; r < 4; r++) ds_store(0.0f, dso, 16 * qh + r);
                }
            } else {
                // The two 16-query halves of the block, one after the other (so that
                // one half's s and dp are live at a time).
                const bool mask = t0 < u0 + KW - 1 || edge;  // crosses the diagonal or an end
#pragma unroll
                for (int qh = 0; qh < 2; qh++) {
                    // the first half when all its 16 queries precede this wave's keys (the
                    // block's second half starts the diagonal): p = ds = 0, stored as such
                    if (qh == 0 && t0 + 16 <= u0) {
                        if (col_ok) {
#pragma unroll
                            for (int r = 0; r < 4; r++) ds_store(0.0f, dso, r);
                        }
                        continue;
                    }
                    // s = Q K^T and dp = dO V^T: two accumulation chains
                    floatx4 sv = {0.f, 0.f, 0.f, 0.f}, dpv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < KS / 4; m++) {
                        const int off = (16 * qh + j) * P + KS * c + 4 * m;
                        const floatx4 qa = *(const floatx4 *)&Qc[off], oa = *(const floatx4 *)&Oc[off];
                        const floatx4 ka = *(const floatx4 *)&Kt[(wave * KW + j) * P + KS * c + 4 * m];
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            sv = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[e], ka[e], sv, 0, 0, 0);
                            dpv = __builtin_amdgcn_mfma_f32_16x16x4f32(oa[e], vf[4 * m + e], dpv, 0, 0, 0);
                        }
                    }
                    // p = 2^(s - lse log2 e) and ds = p (dp - D), in place; the four
                    // queries of a lane's registers are consecutive: one 16-byte read each
                    const floatx4 L4 = *(const floatx4 *)&Lc[16 * qh + 4 * c];
                    const floatx4 D4 = *(const floatx4 *)&Lc[TB + 16 * qh + 4 * c];
                    if (mask) {
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const int tt = t0 + 16 * qh + 4 * c + r;
                            // masked entries take 2^-inf = 0 (a select of the argument, so
                            // that the exponential is not put under a branch; bitwise
                            // operators: no short-circuit branches)
                            const bool off = (tt < u) | (tt >= T) | (u >= T);
                            const float x = off ? -INFINITY : sv[r] * sl2e - L4[r] * LOG2E;
                            const float p = exp2_fast(x);
                            sv[r] = p;
                            dpv[r] = p * (dpv[r] - D4[r]);
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const float p = exp2_fast(sv[r] * sl2e - L4[r] * LOG2E);
                            sv[r] = p;
                            dpv[r] = p * (dpv[r] - D4[r]);
                        }
                    }
                    if (col_ok) {
#pragma unroll
                        for (int r = 0; r < 4; r++) ds_store(dpv[r], dso, 16 * qh + r);
                    }
                    // dv[u][d] += sum_t p[t][u] dO[t][d], dk[u][d] += sum_t ds[t][u] Q[t][d]:
                    // register r is the A operand for the queries 16 qh + 4 c' + r
                    // (c' = 0..3, one per lane group); the B operands are those
                    // queries' rows at head dims NB j .. NB j + NB - 1
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int off = (16 * qh + 4 * c + r) * P + NB * j;
                        float ob[NB], qv[NB];
                        if constexpr (NB == 4) {
                            const floatx4 o4 = *(const floatx4 *)&Oc[off], q4 = *(const floatx4 *)&Qc[off];
#pragma unroll
                            for (int nb = 0; nb < 4; nb++) {
                                ob[nb] = o4[nb];
                                qv[nb] = q4[nb];
                            }
                        } else {
#pragma unroll
                            for (int nb = 0; nb < NB; nb++) {
                                ob[nb] = Oc[off + nb];
                                qv[nb] = Qc[off + nb];
                            }
                        }
#pragma unroll
                        for (int nb = 0; nb < NB; nb++) {
                            dv[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(sv[r], ob[nb], dv[nb], 0, 0, 0);
                            dk[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(dpv[r], qv[nb], dk[nb], 0, 0, 0);
                        }
                    }
                }
            }  // keys after some queries of the block
            loads_done();
            __syncthreads();
        }
        // the next segment's operands go out before this one's results
        const long long nxt = it + (qend - qfirst);
        if (nxt < hi_g) {
            sg = seg_at(nxt);
            request(sg);
        }
        // register r of block nb: key u0 + 4 c + r, head dim NB j + nb
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
        for (int r = 0; r < 4; r++) {
            const int uu = u0 + 4 * c + r;
            if (uu < T) {
                float *const pk = dkb + (long long)uu * krs + NB * j, *const pv = dvb + (long long)uu * krs + NB * j;
                if constexpr (NB == 4) {
                    *(floatx4 *)pk = floatx4{dk[0][r], dk[1][r], dk[2][r], dk[3][r]} * scale;
                    *(floatx4 *)pv = floatx4{dv[0][r], dv[1][r], dv[2][r], dv[3][r]};
                } else {
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        pk[nb] = dk[nb][r] * scale;
                        pv[nb] = dv[nb][r];
                    }
                }
            }
        }
        if (nxt >= hi_g) break;
        it = nxt;
    }  // segments
}

template <int HD>
__global__ __launch_bounds__(BWD_THREADS, 4) void flash_bwd_dkdv_kernel(float *__restrict__ dqkv,
                                                                        float *__restrict__ ws,
                                                                        float *__restrict__ dsout,
                                                                        const float *__restrict__ dout,
                                                                        const float *__restrict__ qkv,
                                                                        const float *__restrict__ lse,
                                                                        const float *__restrict__ Dbuf, int T, int C,
                                                                        int NH, int BH, float scale) {
    dkdv_body<HD>(dqkv, ws, dsout, dout, qkv, lse, Dbuf, T, C, NH, BH, scale);
}

// D[bh][t] = dO_t . O_t over the head's HD dims: HD / 4 consecutive threads
// per (b, t, head), one 16-byte piece of each operand each (coalesced rows,
// many loads in flight), summed across those lanes by DPP exchanges in a
// fixed order.  Every lane takes part in the exchanges; lanes past the end
// contribute zeros and write nothing.
template <int HD>
__global__ __launch_bounds__(256) void flash_bwd_D_kernel(float *__restrict__ Dbuf, const float *__restrict__ dout,
                                                          const float *__restrict__ out, int T, int C, int NH,
                                                          long long rows) {
    constexpr int G = HD / 4;
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const bool ok = i < rows * NH * G;
    const long long r = ok ? i / G : 0;
    const int d4 = (int)(i % G);
    const long long bt = r / NH;
    const int hh = (int)(r % NH);
    float acc = 0.0f;
    if (ok) {
        const floatx4 x = *(const floatx4 *)(dout + bt * C + hh * HD + 4 * d4);
        const floatx4 y = *(const floatx4 *)(out + bt * C + hh * HD + 4 * d4);
        acc = (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
    }
    // sum over the G = 4, 8 or 16 lanes of the row (an aligned quad, half-row
    // or row of 16 lanes): DPP exchanges, every lane active
    acc += dpp_move<0xB1>(acc);
    acc += dpp_move<0x4E>(acc);
    if (G >= 8) acc += dpp_move<0x141>(acc);
    if (G >= 16) acc += dpp_move<0x140>(acc);
    if (ok && d4 == 0) {
        const long long b = bt / T, t = bt % T;
        Dbuf[(b * NH + hh) * T + t] = acc;
    }
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
// (rows of (T + 3) / 4 * 4 floats: 16-byte stores and loads along a row)
size_t ds_floats(int B, int T, int NH) { return ((size_t)B * NH * T * ((T + 3) / 4 * 4) + 63) / 64 * 64; }

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
    if (AuditSink *au = audit_sink()) {
        // item < B NH items: rows item * QBLK .. + QBLK of HD in ws, one lse each in wlse
        const long long BTC = (long long)B * T * C, BHT = (long long)B * NH * T;
        const long long nws = (long long)B * NH * items * QBLK;
        const char *k = HD == 16 ? "flash_fwd_kernel<16>" : HD == 32 ? "flash_fwd_kernel<32>" : "flash_fwd_kernel<64>";
        audit(au, k, "qkv", qkv, 3 * BTC, false);
        audit(au, k, "out", out, BTC, true);
        audit(au, k, "lse", lse, BHT, true);
        audit(au, k, "ws", ws, nws * HD, true);
        audit(au, k, "wlse", wlse, nws, true);
        if (items != (T + QBLK - 1) / QBLK) {
            audit(au, "flash_fwd_merge_kernel", "ws", ws, nws * HD, false);
            audit(au, "flash_fwd_merge_kernel", "wlse", wlse, nws, false);
            audit(au, "flash_fwd_merge_kernel", "out", out, BTC, true);
            audit(au, "flash_fwd_merge_kernel", "lse", lse, BHT, true);
        }
        return hipSuccess;
    }
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
    if (AuditSink *au = audit_sink()) {
        // G workgroups, two partial slots of 2 QBLK HD floats each; ds of every (b, h) T x T
        const long long BTC = (long long)B * T * C, BHT = (long long)B * NH * T;
        const long long G = dkdv_groups(B, T, NH, HD);
        const char *k = HD == 16 ? "flash_bwd_dkdv_kernel<16>" : HD == 32 ? "flash_bwd_dkdv_kernel<32>"
                                                                          : "flash_bwd_dkdv_kernel<64>";
        audit(au, "flash_bwd_D_kernel", "Dbuf", Dbuf, BHT, true);
        audit(au, "flash_bwd_D_kernel", "dout", dout, BTC, false);
        audit(au, "flash_bwd_D_kernel", "out", out, BTC, false);
        audit(au, k, "dqkv", dqkv, 3 * BTC, true);
        audit(au, k, "kvws", ws + ds_floats(B, T, NH), 2 * G * 2 * QBLK * HD, true);
        audit(au, k, "ds", ws, BHT * ((T + 3) / 4 * 4), true);
        audit(au, k, "dout", dout, BTC, false);
        audit(au, k, "qkv", qkv, 3 * BTC, false);
        audit(au, k, "lse", lse, BHT, false);
        audit(au, k, "Dbuf", Dbuf, BHT, false);
        audit(au, "flash_bwd_sum_kernel", "kvws", ws + ds_floats(B, T, NH), 2 * G * 2 * QBLK * HD, false);
        audit(au, "flash_bwd_sum_kernel", "dqkv", dqkv, 3 * BTC, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(flash_bwd_D_kernel<HD>, dim3((unsigned)((rows * NH * (HD / 4) + 255) / 256)), dim3(256), 0, s, Dbuf, dout,
                       out, T, C, NH, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = dkdv_groups(B, T, NH, HD);
    float *ds = ws, *kvws = ws + ds_floats(B, T, NH);
    hipLaunchKernelGGL(flash_bwd_dkdv_kernel<HD>, dim3(G), dim3(BWD_THREADS), 0, s, dqkv, kvws, ds, dout, qkv, lse,
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
