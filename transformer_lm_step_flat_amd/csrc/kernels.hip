// Memory-bound kernels of the training step for gfx950: encoder, LayerNorm,
// causal softmax, fused cross-entropy, reductions, AdamW.  Row kernels give
// each row to one 64-lane wavefront and reduce across lanes with shuffles;
// streaming kernels move 16 bytes per lane per access.  Every reduction runs
// in a fixed order, so results are bitwise reproducible run to run.
#include "audit.h"
#include "common.h"
#include "kernels.h"

namespace {

inline unsigned grid_for(size_t n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

__global__ void fill_kernel(float *p, size_t n, float v) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

// The same for 16-byte-aligned buffers of n4 float4s: each workgroup stores
// one contiguous run of 4 x 256 float4s with non-temporal stores.
__global__ __launch_bounds__(256) void fill4_kernel(floatx4 *p, size_t n4, float v) {
    const size_t base = (size_t)blockIdx.x * 1024 + threadIdx.x;
    const floatx4 x = {v, v, v, v};
#pragma unroll
    for (int u = 0; u < 4; u++)
        if (base + (size_t)u * 256 < n4) __builtin_nontemporal_store(x, p + base + (size_t)u * 256);
}

__global__ void fill_i32_kernel(int32_t *p, size_t n, int32_t v) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

__device__ __forceinline__ int clamp_id(int id, int V) { return id < 0 ? 0 : (id >= V ? V - 1 : id); }

// Id validation and the position order of the embedding backward: the
// positions sorted by (id, position).  One wavefront per position p: its
// rank is the number of positions q with key(q) < key(p), key = id * BT +
// position, each lane counting every 64th q and the lanes' counts summed.
// Keys are distinct (positions differ), so the ranks are a permutation.
__global__ __launch_bounds__(256) void token_prep_kernel(const int32_t *inp, const int32_t *tgt, int32_t *order,
                                                         int32_t *err, int BT, int V) {
    const int lane = threadIdx.x & 63;
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= BT) return;
    const int id = inp[p];
    const long long mykey = (long long)clamp_id(id, V) * BT + p;
    int cnt = 0;
    for (int q = lane; q < BT; q += 64) cnt += (long long)clamp_id(inp[q], V) * BT + q < mykey;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, WAVE);
    if (lane == 0) {
        int e = 0;
        if (id < 0 || id >= V) e |= 1;
        if (tgt) {
            const int tg = tgt[p];
            if (tg < 0 || tg >= V) e |= 2;
        }
        if (e) atomicOr(err, e);
        order[cnt] = p;
    }
}

// The same order in O(BT log BT) work, for large BT.  Pass 1: each
// workgroup sorts one chunk of TCH keys id * BT + position (64-bit, distinct)
// in LDS with a bitonic network (pass (k, j) compares keys i and i + j, i
// having bit j clear, ascending where bit k of i is clear) and stores it.
// Pass 2: a position's rank is the number of smaller keys, summed over the
// sorted chunks by binary search (16 chunks' searches advanced together, so
// that their loads are in flight at once).
constexpr int TCH = 1024;

__global__ __launch_bounds__(512) void token_chunk_sort_kernel(const int32_t *inp, uint64_t *sorted, int BT, int V) {
    __shared__ uint64_t key[TCH];
    const int tid = threadIdx.x, c0 = blockIdx.x * TCH, n = min(TCH, BT - c0);
    for (int i = tid; i < TCH; i += 512)
        key[i] = i < n ? (uint64_t)clamp_id(inp[c0 + i], V) * (uint64_t)BT + (uint64_t)(c0 + i) : ~0ull;
    __syncthreads();
    auto pass = [&](int k, int j) {
        const int i = ((tid & ~(j - 1)) << 1) | (tid & (j - 1)), l = i | j;
        const uint64_t a = key[i], b = key[l];
        if ((a > b) == ((i & k) == 0)) {
            key[i] = b;
            key[l] = a;
        }
    };
    for (int k = 2; k <= TCH; k <<= 1) {
        int j = k >> 1;
        for (; j > 32; j >>= 1) {
            pass(k, j);
            __syncthreads();
        }
        // j <= 32: a wavefront's 64 pairs lie in one block of 128 keys of
        // its own, so only its own accesses need ordering
        for (; j > 0; j >>= 1) {
            pass(k, j);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        __syncthreads();
    }
    for (int i = tid; i < n; i += 512) sorted[c0 + i] = key[i];
}

__global__ __launch_bounds__(256) void token_rank_kernel(const int32_t *inp, const int32_t *tgt, const uint64_t *sorted,
                                                         int32_t *order, int32_t *err, int BT, int V) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= BT) return;
    const int id = inp[p];
    int e = (id < 0 || id >= V) ? 1 : 0;
    if (tgt) {
        const int tg = tgt[p];
        if (tg < 0 || tg >= V) e |= 2;
    }
    if (e) atomicOr(err, e);
    const uint64_t kp = (uint64_t)clamp_id(id, V) * (uint64_t)BT + (uint64_t)p;
    const int nch = (BT + TCH - 1) / TCH;
    int rank = 0;
    constexpr int NB = 16;
    for (int cb = 0; cb < nch; cb += NB) {
        // per chunk: keys below kp lie in [0, b + m) with the first b of them known smaller
        int b[NB], m[NB];
#pragma unroll
        for (int u = 0; u < NB; u++) {
            b[u] = 0;
            m[u] = cb + u < nch ? min(TCH, BT - (cb + u) * TCH) : 0;
        }
        for (int step = 0; step <= 10; step++) {  // ceil(log2(TCH + 1)) halvings
            // all the probes' loads first (in bounds for finished and absent chunks too)
            uint64_t v[NB];
#pragma unroll
            for (int u = 0; u < NB; u++) {
                const int c = min(cb + u, nch - 1);
                v[u] = sorted[c * TCH + (m[u] > 0 ? b[u] + (m[u] >> 1) : 0)];
            }
#pragma unroll
            for (int u = 0; u < NB; u++) {
                const int h = m[u] >> 1;
                const bool less = v[u] < kp;
                b[u] = m[u] > 0 && less ? b[u] + h + 1 : b[u];
                m[u] = m[u] > 0 ? (less ? m[u] - h - 1 : h) : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < NB; u++) rank += b[u];
    }
    order[rank] = p;
}

__global__ void encoder_forward_kernel(float *out, const int32_t *inp, const float *wte, const float *wpe, int T,
                                       int C, int V, long long total4) {
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total4) return;
    const int C4 = C / 4;
    long long bt = i / C4;
    int c4 = (int)(i - bt * C4);
    int t = (int)(bt % T);
    int id = clamp_id(inp[bt], V);
    floatx4 a = ((const floatx4 *)(wte + (long long)id * C))[c4];
    floatx4 b = ((const floatx4 *)(wpe + (long long)t * C))[c4];
    ((floatx4 *)(out + bt * C))[c4] = a + b;
}

// dwte scatter-add in two deterministic phases over the positions sorted by
// (id, position).  Phase 1: the sorted sequence is cut into chunks of
// ENC_CHUNK entries; within a chunk each run of equal ids (a segment) is
// summed in position order and stored at part[first sorted index of the
// segment].  Phase 2: each run of equal ids adds its segments (its first one
// and one per chunk boundary inside the run, in order) to the id's row.  No
// thread adds a run's rows one by one: phase 1 is one round of loads per
// chunk, phase 2 three per ENC_RUN_BATCH chunks of a long run (positions,
// ids, segment sums).
constexpr int ENC_CHUNK = 16;  // a chunk's rows are all requested at once
constexpr int ENC_RUN_BATCH = 8;  // chunk boundaries of a run examined together in phase 2

__global__ __launch_bounds__(64) void encoder_backward_segments_kernel(floatx4 *part, const float *dout,
                                                                        const int32_t *inp, const int32_t *order,
                                                                        int BT, int C, int V) {
    __shared__ int ids[ENC_CHUNK + 1], pos[ENC_CHUNK];
    const int base = blockIdx.x * ENC_CHUNK, n = min(ENC_CHUNK, BT - base);
    const int tid = threadIdx.x;
    if (tid < n) {
        const int p = order[base + tid];
        pos[tid] = p;
        ids[tid] = clamp_id(inp[p], V);
    }
    if (tid == 0) ids[n] = -1;  // closes the last segment
    __syncthreads();
    const int C4 = C / 4, c4 = blockIdx.y * 64 + tid;
    if (c4 >= C4) return;
    const floatx4 *src = (const floatx4 *)dout + c4;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int seg = 0;
    floatx4 v[ENC_CHUNK];
#pragma unroll
    for (int e = 0; e < ENC_CHUNK; e++) v[e] = e < n ? src[(long long)pos[e] * C4] : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < ENC_CHUNK; e++) {
        if (e < n) {
            acc += v[e];
            if (ids[e + 1] != ids[e]) {
                part[(long long)(base + seg) * C4 + c4] = acc;
                acc = floatx4{0.f, 0.f, 0.f, 0.f};
                seg = e + 1;
            }
        }
    }
}

// (one sorted position per workgroup: the position, its id and the run's
// boundaries are the same for the whole wavefront, so their loads are
// scalar loads; most positions are not the first of their run and end
// after two of them)
__global__ __launch_bounds__(64) void encoder_backward_runs_kernel(float *dwte, const floatx4 *part,
                                                                    const int32_t *inp, const int32_t *order, int BT,
                                                                    int C, int V) {
    const int i = blockIdx.x;
    // (loads without short-circuit conditions, so that they issue together)
    const int pc = order[i], pp = order[i > 0 ? i - 1 : 0];
    const int id = clamp_id(inp[pc], V), idp = clamp_id(inp[pp], V);
    if (i > 0 && idp == id) return;  // not the first entry of its run
    const int C4 = C / 4, c4 = blockIdx.y * 64 + threadIdx.x;
    if (c4 >= C4) return;
    floatx4 acc = part[(long long)i * C4 + c4];
    // The run's later segments start at the chunk boundaries inside it (every
    // chunk start below BT holds a segment sum).  The first boundary is
    // examined alone: most runs end before it.  Beyond it the ids at
    // ENC_RUN_BATCH boundaries are requested together, then the segment sums
    // of those still inside the run, added in order.
    int k = (i / ENC_CHUNK + 1) * ENC_CHUNK;
    if (k < BT && clamp_id(inp[order[k]], V) == id) {
        acc += part[(long long)k * C4 + c4];
        k += ENC_CHUNK;
    } else {
        k = BT;
    }
    while (k < BT) {
        int pk[ENC_RUN_BATCH];
#pragma unroll
        for (int u = 0; u < ENC_RUN_BATCH; u++) {
            const int kk = k + u * ENC_CHUNK;
            pk[u] = kk < BT ? order[kk] : 0;
        }
        int idu[ENC_RUN_BATCH];
#pragma unroll
        for (int u = 0; u < ENC_RUN_BATCH; u++) idu[u] = clamp_id(inp[pk[u]], V);
        int n = 0;  // leading boundaries of the batch inside the run
        bool in = true;
#pragma unroll
        for (int u = 0; u < ENC_RUN_BATCH; u++) {
            in = in & (k + u * ENC_CHUNK < BT) & (idu[u] == id);
            n += in ? 1 : 0;
        }
        if (n == 0) break;
        // (indices clamped to the last boundary inside the run: every load is
        // valid and they issue together; only the first n are added)
        floatx4 v[ENC_RUN_BATCH];
#pragma unroll
        for (int u = 0; u < ENC_RUN_BATCH; u++)
            v[u] = part[(long long)(k + min(u, n - 1) * ENC_CHUNK) * C4 + c4];
#pragma unroll
        for (int u = 0; u < ENC_RUN_BATCH; u++)
            if (u < n) acc += v[u];
        if (n < ENC_RUN_BATCH) break;
        k += ENC_RUN_BATCH * ENC_CHUNK;
    }
    floatx4 *dst = (floatx4 *)(dwte + (long long)id * C) + c4;
    *dst = *dst + acc;
}

__global__ void encoder_backward_wpe_kernel(float *dwpe, const float *dout, int B, int T, int C) {
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int C4 = C / 4;
    if (i >= (long long)T * C4) return;
    int t = (int)(i / C4), c4 = (int)(i % C4);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < B; b++) acc += ((const floatx4 *)(dout + ((long long)b * T + t) * C))[c4];
    floatx4 *dst = (floatx4 *)(dwpe + (long long)t * C) + c4;
    *dst = *dst + acc;
}

// LayerNorm forward: one wavefront per row, the row held in registers
// (NV float4 per lane, C <= 256 * NV).
template <int NV>
__global__ __launch_bounds__(256) void layernorm_forward_kernel(float *out, float *mean, float *rstd,
                                                                const float *inp, const float *w,
                                                                const float *b, int N, int C) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= N) return;
    const int C4 = C / 4;
    const floatx4 *x = (const floatx4 *)(inp + (long long)row * C);
    floatx4 v[NV], g[NV], bb[NV];
    // the row and the affine parameters are all requested before the first
    // reduction, so that only one memory latency sits on the row's path
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int k = lane + 64 * i;
        const int kc = k < C4 ? k : C4 - 1;
        v[i] = x[kc];
        g[i] = ((const floatx4 *)w)[kc];
        bb[i] = ((const floatx4 *)b)[kc];
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        if (lane + 64 * i >= C4) v[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        sum += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
    }
    const float m = wave_sum(sum) / C;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        int k = lane + 64 * i;
        if (k < C4) {
            floatx4 d = v[i] - m;
            ss += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
        }
    }
    const float rs = rsqrtf(wave_sum(ss) / C + 1e-5f);
    floatx4 *o = (floatx4 *)(out + (long long)row * C);
#pragma unroll
    for (int i = 0; i < NV; i++) {
        int k = lane + 64 * i;
        if (k < C4) o[k] = (v[i] - m) * rs * g[i] + bb[i];
    }
    if (lane == 0) {
        mean[row] = m;
        rstd[row] = rs;
    }
}

constexpr int COL_CHUNK = 16;  // rows per LayerNorm-backward block (and per partial row)

// whether nw wavefronts' column sums of dw and db fit in 64 KB of LDS together
__host__ __device__ inline bool ln_bwd_one_pass(int nw, int C) { return (size_t)nw * 2 * C * sizeof(float) <= 65536; }

// LayerNorm backward.  Block b takes rows [16b, 16b+16) with nw = 8
// wavefronts (blockDim.x / 64), wavefront w the rows 16b + w + nw k, one at a
// time with the next row's loads issued before the current row's reductions:
//   xhat = (x - mean) rstd, g = dy * w,
//   dx (+)= rstd (g - mean_c(g) - xhat mean_c(g xhat)).
// Per-column sums of dy * xhat and dy are kept per lane, combined over the
// wavefronts in a fixed order and written as the block's partial row
// [dw (C) | db (C)].
template <int NV>
__global__ __launch_bounds__(512) void layernorm_backward_kernel(float *dinp, float *partial, const float *dout,
                                                                 const float *inp, const float *w,
                                                                 const float *mean, const float *rstd, int N, int C,
                                                                 int accumulate) {
    extern __shared__ floatx4 lds4[];  // [nw][2C/4] or [nw][C/4]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int C4 = C / 4;
    floatx4 wv[NV], dwacc[NV], dbacc[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int k = lane + 64 * i;
        wv[i] = k < C4 ? ((const floatx4 *)w)[k] : floatx4{0.f, 0.f, 0.f, 0.f};
        dwacc[i] = dbacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    const int r0 = blockIdx.x * COL_CHUNK + wave;
    if constexpr (NV <= 4) {
        floatx4 xn[NV], dn[NV], on[NV] = {};
        float mun = 0.f, rsn = 0.f;
        // The loads read only valid addresses (a row past the end is never used,
        // lanes past the row end read its last float4) and the zeros of lanes
        // past the row end are applied when the row is used, so the next row's
        // loads stay in flight while the current row is reduced.
        auto fetch = [&](int row) {
            const int rr = row < N ? row : N - 1;
            const floatx4 *x = (const floatx4 *)(inp + (long long)rr * C);
            const floatx4 *dy = (const floatx4 *)(dout + (long long)rr * C);
            const floatx4 *dx = (const floatx4 *)(dinp + (long long)rr * C);
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const int k = lane + 64 * i, kc = k < C4 ? k : C4 - 1;
                xn[i] = x[kc];
                dn[i] = dy[kc];
                if (accumulate) on[i] = dx[kc];
            }
            mun = mean[rr];
            rsn = rstd[rr];
        };
        fetch(r0);
        for (int k = 0; k < COL_CHUNK / nw; k++) {
            const int row = r0 + nw * k;
            if (row >= N) break;
            floatx4 xc[NV], dc[NV], oc[NV];
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const bool kk = lane + 64 * i < C4;
                xc[i] = kk ? xn[i] : z4;
                dc[i] = kk ? dn[i] : z4;
                oc[i] = (kk && accumulate) ? on[i] : z4;
            }
            const float mu = mun, rs = rsn;
            // prefetch the next row while reducing this one (wide rows: registers
            // would spill, so they load each row when it is reached)
            constexpr bool kPrefetch = NV <= 4;
            if (kPrefetch && k + 1 < COL_CHUNK / nw) fetch(row + nw);
            floatx4 xh[NV], g[NV];
            float sg = 0.f, sgx = 0.f;
#pragma unroll
            for (int i = 0; i < NV; i++) {
                xh[i] = (xc[i] - mu) * rs;
                g[i] = dc[i] * wv[i];
                const floatx4 gx = g[i] * xh[i];
                sg += (g[i][0] + g[i][1]) + (g[i][2] + g[i][3]);
                sgx += (gx[0] + gx[1]) + (gx[2] + gx[3]);
                dwacc[i] += dc[i] * xh[i];
                dbacc[i] += dc[i];
            }
            const float mg = wave_sum(sg) / C, mgx = wave_sum(sgx) / C;
            floatx4 *dx = (floatx4 *)(dinp + (long long)row * C);
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const int kk = lane + 64 * i;
                if (kk < C4) dx[kk] = oc[i] + rs * (g[i] - mg - xh[i] * mgx);
            }
            if (!kPrefetch && k + 1 < COL_CHUNK / nw) fetch(row + nw);
        }
    } else {
        // Wide rows: only x and dy of the next row are prefetched, the
        // affine weight is read again per row (from cache) and dx is read
        // where it is written, so that the row state fits without spills.
        floatx4 xn[NV], dn[NV];
        float mun = 0.f, rsn = 0.f;
        auto fetch = [&](int row) {
            const int rr = row < N ? row : N - 1;
            const floatx4 *x = (const floatx4 *)(inp + (long long)rr * C);
            const floatx4 *dy = (const floatx4 *)(dout + (long long)rr * C);
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const int k = lane + 64 * i, kc = k < C4 ? k : C4 - 1;
                xn[i] = x[kc];
                dn[i] = dy[kc];
            }
            mun = mean[rr];
            rsn = rstd[rr];
        };
        fetch(r0);
        for (int k = 0; k < COL_CHUNK / nw; k++) {
            const int row = r0 + nw * k;
            if (row >= N) break;
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            floatx4 xh[NV], g[NV];
            const float mu = mun, rs = rsn;
            float sg = 0.f, sgx = 0.f;
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const int kk = lane + 64 * i;
                const bool in = kk < C4;
                const floatx4 d = in ? dn[i] : z4;
                xh[i] = in ? (xn[i] - mu) * rs : z4;
                g[i] = d * (in ? ((const floatx4 *)w)[kk] : z4);
                const floatx4 gx = g[i] * xh[i];
                sg += (g[i][0] + g[i][1]) + (g[i][2] + g[i][3]);
                sgx += (gx[0] + gx[1]) + (gx[2] + gx[3]);
                dwacc[i] += d * xh[i];
                dbacc[i] += d;
            }
            if (k + 1 < COL_CHUNK / nw) fetch(row + nw);
            const float mg = wave_sum(sg) / C, mgx = wave_sum(sgx) / C;
            floatx4 *dx = (floatx4 *)(dinp + (long long)row * C);
#pragma unroll
            for (int i = 0; i < NV; i++) {
                const int kk = lane + 64 * i;
                if (kk < C4) {
                    const floatx4 v = rs * (g[i] - mg - xh[i] * mgx);
                    dx[kk] = accumulate ? dx[kk] + v : v;
                }
            }
        }
    }
    // the wavefronts' column sums are combined in a fixed order through LDS:
    // [nw][2C] at once where that fits in 64 KB, else in two passes through
    // [nw][C] (the dw half, then the db half)
    floatx4 *out = (floatx4 *)(partial + (long long)blockIdx.x * 2 * C);
    if (ln_bwd_one_pass(nw, C)) {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int k = lane + 64 * i;
            if (k < C4) {
                lds4[wave * 2 * C4 + k] = dwacc[i];
                lds4[wave * 2 * C4 + C4 + k] = dbacc[i];
            }
        }
        __syncthreads();
        for (int c = threadIdx.x; c < 2 * C4; c += blockDim.x) {
            floatx4 t = lds4[c];
            for (int q = 1; q < nw; q++) t += lds4[q * 2 * C4 + c];
            out[c] = t;
        }
        return;
    }
#pragma unroll
    for (int half = 0; half < 2; half++) {
        if (half) __syncthreads();  // the dw half has been read
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int k = lane + 64 * i;
            if (k < C4) lds4[wave * C4 + k] = half ? dbacc[i] : dwacc[i];
        }
        __syncthreads();
        for (int c = threadIdx.x; c < C4; c += blockDim.x) {
            floatx4 t = lds4[c];
            for (int q = 1; q < nw; q++) t += lds4[q * C4 + c];
            out[half * C4 + c] = t;
        }
    }
}

// dst[i] (+)= sum_{p < P} src[p*ld + i], 4 consecutive i per thread, p in order.
__global__ __launch_bounds__(256) void sum_partials_kernel(float *dst, const float *src, int P, size_t n4,
                                                           size_t ld4, int accumulate) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const floatx4 *s4 = (const floatx4 *)src;
    floatx4 acc = s4[i];
    for (int p = 1; p < P; p++) acc += s4[(size_t)p * ld4 + i];
    floatx4 *d4 = (floatx4 *)dst;
    d4[i] = accumulate ? d4[i] + acc : acc;
}

// Two split-K sums in one launch: dst1[i] (+)= sum_p src1[p*n1 + i] for the
// first n1 (float4) threads, the same for region 2 after them; p in order,
// the loads of up to 8 partials issued before the adds.
__global__ __launch_bounds__(256) void sum_partials2_kernel(floatx4 *dst1, const floatx4 *src1, size_t n1,
                                                            floatx4 *dst2, const floatx4 *src2, size_t n2, int P,
                                                            int accumulate) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    floatx4 *dst = dst1;
    const floatx4 *src = src1;
    size_t ld = n1;
    if (i >= n1) {
        i -= n1;
        if (i >= n2) return;
        dst = dst2;
        src = src2;
        ld = n2;
    }
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int p = 0;
    for (; p + 8 <= P; p += 8) {
        floatx4 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = src[(size_t)(p + u) * ld + i];
#pragma unroll
        for (int u = 0; u < 8; u++) acc += v[u];
    }
    for (; p < P; p++) acc += src[(size_t)p * ld + i];
    dst[i] = accumulate ? dst[i] + acc : acc;
}

// The split-K sums of one weight-gradient site over all L layers in one
// launch: for layer l, dst1[l*n1 + i] += sum_p src1[(l*P + p)*n1 + i] and the
// same for region 2 (n counted in float4s; p in order).
__global__ __launch_bounds__(256) void sum_layers_kernel(floatx4 *dst1, const floatx4 *src1, size_t n1,
                                                         floatx4 *dst2, const floatx4 *src2, size_t n2, int P,
                                                         int L) {
    const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t per = n1 + n2;
    if (g >= per * L) return;
    const size_t l = g / per;
    size_t i = g % per;
    floatx4 *dst;
    const floatx4 *src;
    size_t ld;
    if (i < n1) {
        dst = dst1 + l * n1;
        src = src1 + l * P * n1;
        ld = n1;
    } else {
        i -= n1;
        dst = dst2 + l * n2;
        src = src2 + l * P * n2;
        ld = n2;
    }
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int p = 0;
    for (; p + 8 <= P; p += 8) {
        floatx4 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = src[(size_t)(p + u) * ld + i];
#pragma unroll
        for (int u = 0; u < 8; u++) acc += v[u];
    }
    for (; p < P; p++) acc += src[(size_t)p * ld + i];
    dst[i] = dst[i] + acc;
}

// dst (n floats) and dst2 (n2 floats) += the column sums of partial rows of
// n + n2 floats (fixed order): used for the [dw | db] partials of LayerNorm.
// sum of src[p * ld] over p = p0, p0 + 16, ... < P, added in that order; the
// loads are issued sixteen (then eight) at a time so that their latencies
// overlap.
__device__ __forceinline__ floatx4 sum_rows_strided(const floatx4 *src, int p0, int P, size_t ld) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int p = p0;
    for (; p + 16 * 15 < P; p += 16 * 16) {
        floatx4 v[16];
#pragma unroll
        for (int u = 0; u < 16; u++) v[u] = src[(size_t)(p + 16 * u) * ld];
#pragma unroll
        for (int u = 0; u < 16; u++) acc += v[u];
    }
    for (; p + 16 * 7 < P; p += 16 * 8) {
        floatx4 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = src[(size_t)(p + 16 * u) * ld];
#pragma unroll
        for (int u = 0; u < 8; u++) acc += v[u];
    }
    for (; p < P; p += 16) acc += src[(size_t)p * ld];
    return acc;
}

__global__ __launch_bounds__(256) void sum_partials_split_kernel(float *dst, float *dst2, const float *src, int P,
                                                                 int n4, int n24) {
    __shared__ floatx4 lds[16][16];
    const int c = threadIdx.x & 15, pl = threadIdx.x >> 4;
    const int i = blockIdx.x * 16 + c, ld4 = n4 + n24;
    const floatx4 *s4 = (const floatx4 *)src;
    const floatx4 acc = i < ld4 ? sum_rows_strided(s4 + i, pl, P, (size_t)ld4) : floatx4{0.f, 0.f, 0.f, 0.f};
    lds[pl][c] = acc;
    __syncthreads();
    if (pl == 0 && i < ld4) {
        floatx4 t = lds[0][c];
#pragma unroll
        for (int k = 1; k < 16; k++) t += lds[k][c];
        floatx4 *d4 = i < n4 ? (floatx4 *)dst + i : (floatx4 *)dst2 + (i - n4);
        *d4 = *d4 + t;
    }
}

// The LayerNorm parameter sums of a whole backward pass in one launch: slot
// y = blockIdx.y holds P partial rows [dw | db] of one LayerNorm; slots
// [0, L) are the ln1 of each layer, [L, 2L) the ln2, 2L the final one, each
// added into its (w, b) gradient at stride C within its group.
__global__ __launch_bounds__(256) void ln_param_sums_kernel(float *w1, float *b1, float *w2, float *b2, float *w3,
                                                            float *b3, int L, const float *partial, int P, int C) {
    __shared__ floatx4 lds[16][16];
    const int y = blockIdx.y;
    const int c = threadIdx.x & 15, pl = threadIdx.x >> 4;
    const int C4 = C / 4, i = blockIdx.x * 16 + c, ld4 = 2 * C4;
    const floatx4 *s4 = (const floatx4 *)(partial + (size_t)y * P * 2 * C);
    const floatx4 acc = i < ld4 ? sum_rows_strided(s4 + i, pl, P, (size_t)ld4) : floatx4{0.f, 0.f, 0.f, 0.f};
    lds[pl][c] = acc;
    __syncthreads();
    if (pl == 0 && i < ld4) {
        floatx4 t = lds[0][c];
#pragma unroll
        for (int k = 1; k < 16; k++) t += lds[k][c];
        float *w = y < L ? w1 + (size_t)y * C : (y < 2 * L ? w2 + (size_t)(y - L) * C : w3);
        float *b = y < L ? b1 + (size_t)y * C : (y < 2 * L ? b2 + (size_t)(y - L) * C : b3);
        floatx4 *d4 = i < C4 ? (floatx4 *)w + i : (floatx4 *)b + (i - C4);
        *d4 = *d4 + t;
    }
}

// The same for many partials: 16 float4 columns x 16 partial lanes per block;
// lane l sums p = l, l+16, ...; the 16 lane sums are added in a fixed order.
__global__ __launch_bounds__(256) void sum_partials_wide_kernel(float *dst, const float *src, int P, size_t n4,
                                                                size_t ld4, int accumulate) {
    __shared__ floatx4 lds[16][16];
    const int c = threadIdx.x & 15, pl = threadIdx.x >> 4;
    const size_t i = (size_t)blockIdx.x * 16 + c;
    const floatx4 *s4 = (const floatx4 *)src;
    const floatx4 acc = i < n4 ? sum_rows_strided(s4 + i, pl, P, ld4) : floatx4{0.f, 0.f, 0.f, 0.f};
    lds[pl][c] = acc;
    __syncthreads();
    if (pl == 0 && i < n4) {
        floatx4 t = lds[0][c];
#pragma unroll
        for (int k = 1; k < 16; k++) t += lds[k][c];
        floatx4 *d4 = (floatx4 *)dst;
        d4[i] = accumulate ? d4[i] + t : t;
    }
}

constexpr int SM_NV = 16;  // up to 1024 columns per row in registers

__device__ __forceinline__ int pad_end(int t, int T) {
    int e = (t / CAUSAL_PAD + 1) * CAUSAL_PAD;
    return e < T ? e : T;
}

// Causal softmax of one row per wavefront, in place.
__global__ __launch_bounds__(256) void attn_softmax_forward_kernel(float *att, long long nrows, int T) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= nrows) return;
    const int t = (int)(row % T);
    float *r = att + row * T;
    float x[SM_NV];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < SM_NV; i++) {
        int u = lane + 64 * i;
        x[i] = u <= t ? r[u] : -INFINITY;
        mx = fmaxf(mx, x[i]);
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < SM_NV; i++) {
        int u = lane + 64 * i;
        x[i] = u <= t ? __expf(x[i] - mx) : 0.f;
        sum += x[i];
    }
    const float inv = 1.0f / wave_sum(sum);
    const int e = pad_end(t, T);
#pragma unroll
    for (int i = 0; i < SM_NV; i++) {
        int u = lane + 64 * i;
        if (u < e) r[u] = x[i] * inv;
    }
}

// dS[t][u] = P[t][u] (dP[t][u] - sum_u' P[t][u'] dP[t][u']) for u <= t, in place over dP.
__global__ __launch_bounds__(256) void attn_softmax_backward_kernel(float *dp, const float *att, long long nrows,
                                                                    int T) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= nrows) return;
    const int t = (int)(row % T);
    float *d = dp + row * T;
    const float *pr = att + row * T;
    float pv[SM_NV], dv[SM_NV];
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < SM_NV; i++) {
        int u = lane + 64 * i;
        pv[i] = u <= t ? pr[u] : 0.f;
        dv[i] = u <= t ? d[u] : 0.f;
        dot += pv[i] * dv[i];
    }
    dot = wave_sum(dot);
    const int e = pad_end(t, T);
#pragma unroll
    for (int i = 0; i < SM_NV; i++) {
        int u = lane + 64 * i;
        if (u < e) d[u] = pv[i] * (dv[i] - dot);
    }
}

__device__ __forceinline__ void online_combine(float &m, float &s, float m2, float s2) {
    float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
    m = mn;
}

// Fused softmax cross-entropy, one 256-thread block per row.  Pass 1: running
// (max, sum of exp) per thread over the V real columns, combined across the
// block.  Pass 2: overwrite the row with (p - onehot) * dscale.
__global__ __launch_bounds__(256) void crossentropy_kernel(float *logits, float *losses, const int32_t *tgt,
                                                           int V, int Vp, float dscale, const int32_t *gate) {
    __shared__ float sm[4], ss[4];
    const int row = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float *z = logits + (long long)row * Vp;
    if (gate && *gate) {  // a bad id in the batch: zero loss gradient
        for (int v4 = threadIdx.x; v4 * 4 < Vp; v4 += 256) ((floatx4 *)z)[v4] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (threadIdx.x == 0) losses[row] = __builtin_nanf("");
        return;
    }
    float m = -INFINITY, s = 0.f;
    for (int v4 = threadIdx.x; v4 * 4 < V; v4 += 256) {
        floatx4 x = ((const floatx4 *)z)[v4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            if (v4 * 4 + e < V) {
                float xe = x[e];
                if (xe > m) {
                    s = s * __expf(m - xe) + 1.0f;
                    m = xe;
                } else {
                    s += __expf(xe - m);
                }
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        float m2 = __shfl_xor(m, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
        online_combine(m, s, m2, s2);
    }
    if (lane == 0) {
        sm[wave] = m;
        ss[wave] = s;
    }
    __syncthreads();
    m = sm[0];
    s = ss[0];
    for (int w = 1; w < 4; w++) online_combine(m, s, sm[w], ss[w]);
    const float lse = m + __logf(s);
    const int y = clamp_id(tgt[row], V);
    if (threadIdx.x == 0) losses[row] = lse - z[y];
    __syncthreads();  // z[y] is read above before any thread overwrites it
    for (int v4 = threadIdx.x; v4 * 4 < Vp; v4 += 256) {
        floatx4 x = ((const floatx4 *)z)[v4];
        floatx4 o;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            int v = v4 * 4 + e;
            o[e] = v < V ? (__expf(x[e] - lse) - (v == y ? 1.0f : 0.0f)) * dscale : 0.0f;
        }
        ((floatx4 *)z)[v4] = o;
    }
}

// The same with the whole row held in registers, for Vp <= 4 * 1024 * NV4:
// one 1024-thread workgroup per row, thread i holding float4s i + 1024 j.
// The row is read once and written once (no second read pass).  Max and sum
// are reduced over the block in a fixed order.
template <int NV4>
__global__ __launch_bounds__(1024) void crossentropy_reg_kernel(float *logits, float *losses, const int32_t *tgt,
                                                                int V, int Vp, float dscale, const int32_t *gate) {
    __shared__ float red[16];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    floatx4 *z = (floatx4 *)(logits + (long long)row * Vp);
    const int n4 = Vp / 4;
    if (gate && *gate) {  // a bad id in the batch: zero loss gradient
        for (int i = tid; i < n4; i += 1024) z[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (tid == 0) losses[row] = __builtin_nanf("");
        return;
    }
    const int y = clamp_id(tgt[row], V);
    floatx4 x[NV4];
#pragma unroll
    for (int j = 0; j < NV4; j++) {
        const int i = tid + 1024 * j;
        x[j] = i < n4 ? z[i] : floatx4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    // the thread holding the target's logit keeps it (other threads overwrite
    // the row in memory before that thread writes the loss)
    const int yown = (y >> 2) % 1024, yj = (y >> 2) / 1024, ye = y & 3;
    float zy = 0.0f;
    if (tid == yown) {
#pragma unroll
        for (int j = 0; j < NV4; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) zy = (j == yj && e == ye) ? x[j][e] : zy;
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NV4; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int v = 4 * (tid + 1024 * j) + e;
            if (v >= V) x[j][e] = -INFINITY;  // padded columns take no part
            m = fmaxf(m, x[j][e]);
        }
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < 16; w++) m = fmaxf(m, red[w]);
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NV4; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) sum += __expf(x[j][e] - m);
    sum = wave_sum(sum);
    __syncthreads();  // every wave has read red[] for the max
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    sum = red[0];
#pragma unroll
    for (int w = 1; w < 16; w++) sum += red[w];
    const float lse = m + __logf(sum);
    if (tid == yown) losses[row] = lse - zy;
#pragma unroll
    for (int j = 0; j < NV4; j++) {
        const int i = tid + 1024 * j;
        if (i < n4) {
            floatx4 o;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int v = 4 * i + e;
                o[e] = (__expf(x[j][e] - lse) - (v == y ? 1.0f : 0.0f)) * dscale;  // 0 for padded columns
            }
            z[i] = o;
        }
    }
}

// loss[0] = mean of losses[0..n): 1024 threads, four loads in flight per
// thread per round, wavefront sums by lane exchanges, then the 16 wavefront
// sums in order.
__global__ __launch_bounds__(1024) void mean_kernel(float *loss, const float *losses, int n) {
    __shared__ float part[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int i = tid; i < n; i += 4096) {
        const float v0 = losses[i];
        const float v1 = i + 1024 < n ? losses[i + 1024] : 0.f;
        const float v2 = i + 2048 < n ? losses[i + 2048] : 0.f;
        const float v3 = i + 3072 < n ? losses[i + 3072] : 0.f;
        a0 += v0;
        a1 += v1;
        a2 += v2;
        a3 += v3;
    }
    const float w = wave_sum((a0 + a1) + (a2 + a3));
    if (lane == 0) part[wave] = w;
    __syncthreads();
    if (wave == 0) {
        const float t = wave_sum(lane < 16 ? part[lane] : 0.f);
        if (lane == 0) loss[0] = t / n;
    }
}

__global__ __launch_bounds__(256) void gelu_forward_kernel(floatx4 *out, const floatx4 *inp, size_t n4) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    floatx4 x = inp[i], y;
#pragma unroll
    for (int e = 0; e < 4; e++) y[e] = gelu_fwd(x[e]);
    out[i] = y;
}

__global__ __launch_bounds__(256) void gelu_backward_kernel(floatx4 *dinp, const floatx4 *inp, const floatx4 *dout,
                                                            size_t n4) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    floatx4 x = inp[i], d = dout[i], y;
#pragma unroll
    for (int e = 0; e < 4; e++) y[e] = d[e] * gelu_grad(x[e]);
    dinp[i] = y;
}

// Each workgroup updates one contiguous run of 4 x 256 float4s: every load
// of the run is issued before any arithmetic, and the four streams are read
// and written with non-temporal hints (each byte is touched once per step).
constexpr int ADAMW_U = 4;
__global__ __launch_bounds__(256) void adamw_kernel(floatx4 *params, const floatx4 *grads, floatx4 *m, floatx4 *v,
                                                    size_t n4, float lr, float b1, float b2, float eps, float wd,
                                                    float inv_c1, float inv_c2, const int32_t *gate) {
    if (gate && *gate) return;  // the batch had an out-of-range id: no update
    const size_t base = (size_t)blockIdx.x * 256 * ADAMW_U + threadIdx.x;
    floatx4 g[ADAMW_U], mm[ADAMW_U], vv[ADAMW_U], p[ADAMW_U];
#pragma unroll
    for (int u = 0; u < ADAMW_U; u++) {
        const size_t i = base + (size_t)u * 256;
        if (i < n4) {
            g[u] = __builtin_nontemporal_load(grads + i);
            mm[u] = __builtin_nontemporal_load(m + i);
            vv[u] = __builtin_nontemporal_load(v + i);
            p[u] = __builtin_nontemporal_load(params + i);
        }
    }
#pragma unroll
    for (int u = 0; u < ADAMW_U; u++) {
        const size_t i = base + (size_t)u * 256;
        if (i < n4) {
            mm[u] = b1 * mm[u] + (1.0f - b1) * g[u];
            vv[u] = b2 * vv[u] + (1.0f - b2) * g[u] * g[u];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float mhat = mm[u][e] * inv_c1, vhat = vv[u][e] * inv_c2;
                p[u][e] -= lr * (mhat / (sqrtf(vhat) + eps) + wd * p[u][e]);
            }
            __builtin_nontemporal_store(mm[u], m + i);
            __builtin_nontemporal_store(vv[u], v + i);
            __builtin_nontemporal_store(p[u], params + i);
        }
    }
}

}  // namespace

hipError_t k_fill(float *p, size_t n, float v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (AuditSink *au = audit_sink()) {
        audit(au, "fill_kernel", "p", p, (long long)n, true);
        return hipSuccess;
    }
    if (n % 4 == 0 && ((uintptr_t)p & 15) == 0 && n / 4 / 1024 < 0x7fffffff) {
        hipLaunchKernelGGL(fill4_kernel, dim3((unsigned)((n / 4 + 1023) / 1024)), dim3(256), 0, s, (floatx4 *)p, n / 4,
                           v);
        return hipGetLastError();
    }
    unsigned g = grid_for(n, 256);
    if (g > 16384) g = 16384;
    hipLaunchKernelGGL(fill_kernel, dim3(g), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t k_fill_i32(int32_t *p, size_t n, int32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (AuditSink *au = audit_sink()) {
        audit(au, "fill_i32_kernel", "p", p, (long long)n, true);
        return hipSuccess;
    }
    unsigned g = grid_for(n, 256);
    if (g > 16384) g = 16384;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(g), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

// The rank kernel is the faster one up to this many positions (measured:
// 13 us at BT = 4096, and 100 us against 20 at 16384).
constexpr int TOKEN_SORT_MIN_BT = 8192;

size_t k_token_prep_work(int BT) { return BT >= TOKEN_SORT_MIN_BT ? 2 * (size_t)BT : 0; }

const char *k_token_prep_name(int BT) { return BT >= TOKEN_SORT_MIN_BT ? "token_rank_kernel" : "token_prep_kernel"; }

hipError_t k_token_prep(const int32_t *inp, const int32_t *tgt, int32_t *order, int32_t *err, int32_t *work, int BT,
                        int V, hipStream_t s) {
    if (BT <= 0 || V <= 0 || (BT >= TOKEN_SORT_MIN_BT && (!work || ((uintptr_t)work & 7)))) return hipErrorInvalidValue;
    const bool sort = BT >= TOKEN_SORT_MIN_BT;
    if (AuditSink *au = audit_sink()) {
        const char *k = k_token_prep_name(BT);
        // every position reads all ids (or the sorted chunks); its rank (an index < BT) receives it
        audit(au, k, "inp", inp, BT, false);
        audit(au, k, "tgt", tgt, BT, false);
        audit(au, k, "order", order, BT, true);
        audit(au, k, "err", err, 1, true);
        if (sort) audit(au, "token_chunk_sort_kernel", "sorted", work, 2LL * BT, true);
        return hipSuccess;
    }
    if (sort) {
        uint64_t *sorted = (uint64_t *)work;
        hipLaunchKernelGGL(token_chunk_sort_kernel, dim3((unsigned)((BT + TCH - 1) / TCH)), dim3(512), 0, s, inp,
                           sorted, BT, V);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(token_rank_kernel, dim3(grid_for(BT, 256)), dim3(256), 0, s, inp, tgt,
                           (const uint64_t *)sorted, order, err, BT, V);
    } else {
        hipLaunchKernelGGL(token_prep_kernel, dim3(grid_for(BT, 4)), dim3(256), 0, s, inp, tgt, order, err, BT, V);
    }
    return hipGetLastError();
}

hipError_t k_encoder_forward(float *out, const int32_t *inp, const float *wte, const float *wpe, int B, int T,
                             int C, int V, hipStream_t s) {
    long long total4 = (long long)B * T * (C / 4);
    if (AuditSink *au = audit_sink()) {
        // ids are clamped to [0, V): wte rows < V; positions t < T
        audit(au, "encoder_forward_kernel", "out", out, (long long)B * T * C, true);
        audit(au, "encoder_forward_kernel", "inp", inp, (long long)B * T, false);
        audit(au, "encoder_forward_kernel", "wte", wte, (long long)V * C, false);
        audit(au, "encoder_forward_kernel", "wpe", wpe, (long long)T * C, false);
        return hipSuccess;
    }
    hipLaunchKernelGGL(encoder_forward_kernel, dim3(grid_for(total4, 256)), dim3(256), 0, s, out, inp, wte, wpe,
                       T, C, V, total4);
    return hipGetLastError();
}

hipError_t k_encoder_backward(float *dwte, float *dwpe, float *part, const float *dout, const int32_t *inp,
                              const int32_t *order, int B, int T, int C, int V, hipStream_t s) {
    const int BT = B * T;
    if (C % 4 || ((uintptr_t)part & 15)) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        // segment sums at sorted index < BT; positions and ids < BT; rows of
        // dwte at clamped ids < V; rows of dwpe at t < T
        const long long BTC = (long long)BT * C;
        audit(au, "encoder_backward_segments_kernel", "part", part, BTC, true);
        audit(au, "encoder_backward_segments_kernel", "dout", dout, BTC, false);
        audit(au, "encoder_backward_segments_kernel", "inp", inp, BT, false);
        audit(au, "encoder_backward_segments_kernel", "order", order, BT, false);
        audit(au, "encoder_backward_runs_kernel", "dwte", dwte, (long long)V * C, true);
        audit(au, "encoder_backward_runs_kernel", "part", part, BTC, false);
        audit(au, "encoder_backward_runs_kernel", "inp", inp, BT, false);
        audit(au, "encoder_backward_runs_kernel", "order", order, BT, false);
        audit(au, "encoder_backward_wpe_kernel", "dwpe", dwpe, (long long)T * C, true);
        audit(au, "encoder_backward_wpe_kernel", "dout", dout, BTC, false);
        return hipSuccess;
    }
    hipLaunchKernelGGL(encoder_backward_segments_kernel, dim3(grid_for(BT, ENC_CHUNK), grid_for(C / 4, 64)), dim3(64), 0,
                       s, (floatx4 *)part, dout, inp, order, BT, C, V);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(encoder_backward_runs_kernel, dim3(BT, grid_for(C / 4, 64)), dim3(64), 0, s, dwte,
                       (const floatx4 *)part, inp, order, BT, C, V);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(encoder_backward_wpe_kernel, dim3(grid_for((size_t)T * (C / 4), 256)), dim3(256), 0, s,
                       dwpe, dout, B, T, C);
    return hipGetLastError();
}

#define LN_DISPATCH(NVV, KER, ...)                                                            \
    switch (NVV) {                                                                              \
        case 1: hipLaunchKernelGGL(KER<1>, __VA_ARGS__); break;                               \
        case 2: hipLaunchKernelGGL(KER<2>, __VA_ARGS__); break;                               \
        case 3: hipLaunchKernelGGL(KER<3>, __VA_ARGS__); break;                               \
        case 4: hipLaunchKernelGGL(KER<4>, __VA_ARGS__); break;                               \
        case 5: hipLaunchKernelGGL(KER<5>, __VA_ARGS__); break;                               \
        case 6: hipLaunchKernelGGL(KER<6>, __VA_ARGS__); break;                               \
        case 7: hipLaunchKernelGGL(KER<7>, __VA_ARGS__); break;                               \
        case 8: hipLaunchKernelGGL(KER<8>, __VA_ARGS__); break;                               \
        default: return hipErrorInvalidValue;                                                   \
    }

hipError_t k_layernorm_forward(float *out, float *mean, float *rstd, const float *inp, const float *w,
                               const float *b, int N, int C, hipStream_t s) {
    if (C % 4 || C > 2048) return hipErrorInvalidValue;
    int nv = (C / 4 + 63) / 64;
    if (nv < 1 || nv > 8) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        const long long NC = (long long)N * C;
        audit(au, "layernorm_forward_kernel", "out", out, NC, true);
        audit(au, "layernorm_forward_kernel", "mean", mean, N, true);
        audit(au, "layernorm_forward_kernel", "rstd", rstd, N, true);
        audit(au, "layernorm_forward_kernel", "inp", inp, NC, false);
        audit(au, "layernorm_forward_kernel", "w", w, C, false);
        audit(au, "layernorm_forward_kernel", "b", b, C, false);
        return hipSuccess;
    }
    LN_DISPATCH(nv, layernorm_forward_kernel, dim3(grid_for(N, 4)), dim3(256), 0, s, out, mean, rstd, inp, w, b, N,
                C);
    return hipGetLastError();
}

int ln_partials(int N) { return (N + COL_CHUNK - 1) / COL_CHUNK; }

hipError_t k_ln_param_sums(float *w1, float *b1, float *w2, float *b2, float *w3, float *b3, int L,
                           const float *partial, int N, int C, hipStream_t s) {
    if (C % 4) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        // 2L + 1 slots of P partial rows of 2C; per layer groups of C
        const long long P = ln_partials(N);
        audit(au, "ln_param_sums_kernel", "partial", partial, (2LL * L + 1) * P * 2 * C, false);
        audit(au, "ln_param_sums_kernel", "w1", w1, (long long)L * C, true);
        audit(au, "ln_param_sums_kernel", "b1", b1, (long long)L * C, true);
        audit(au, "ln_param_sums_kernel", "w2", w2, (long long)L * C, true);
        audit(au, "ln_param_sums_kernel", "b2", b2, (long long)L * C, true);
        audit(au, "ln_param_sums_kernel", "w3", w3, C, true);
        audit(au, "ln_param_sums_kernel", "b3", b3, C, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(ln_param_sums_kernel, dim3(grid_for(2 * C / 4, 16), 2 * L + 1), dim3(256), 0, s, w1, b1, w2, b2,
                       w3, b3, L, partial, ln_partials(N), C);
    return hipGetLastError();
}

hipError_t k_layernorm_backward(float *dinp, float *dw, float *db, float *partial, const float *dout,
                                const float *inp, const float *w, const float *mean, const float *rstd, int N,
                                int C, bool accumulate, hipStream_t s) {
    if (C % 4 || C > 2048) return hipErrorInvalidValue;
    int nv = (C / 4 + 63) / 64;
    const int P = ln_partials(N);
    // eight wavefronts per block (two rows each); their column sums pass
    // through nw x 2C floats of LDS, or nw x C in two passes (C <= 2048: at
    // most 64 KB)
    const int nw = 8;
    const size_t lds = (size_t)nw * (ln_bwd_one_pass(nw, C) ? 2 : 1) * C * sizeof(float);
    if (nv < 1 || nv > 8) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        // rows are clamped to N - 1; block x writes partial row x (P rows of 2C)
        const long long NC = (long long)N * C;
        audit(au, "layernorm_backward_kernel", "dinp", dinp, NC, true);
        audit(au, "layernorm_backward_kernel", "partial", partial, (long long)P * 2 * C, true);
        audit(au, "layernorm_backward_kernel", "dout", dout, NC, false);
        audit(au, "layernorm_backward_kernel", "inp", inp, NC, false);
        audit(au, "layernorm_backward_kernel", "w", w, C, false);
        audit(au, "layernorm_backward_kernel", "mean", mean, N, false);
        audit(au, "layernorm_backward_kernel", "rstd", rstd, N, false);
        if (dw) {
            audit(au, "sum_partials_split_kernel", "partial", partial, (long long)P * 2 * C, false);
            audit(au, "sum_partials_split_kernel", "dw", dw, C, true);
            audit(au, "sum_partials_split_kernel", "db", db, C, true);
        }
        return hipSuccess;
    }
    LN_DISPATCH(nv, layernorm_backward_kernel, dim3(P), dim3(64 * nw), lds, s, dinp, partial, dout, inp, w, mean,
                rstd, N, C, accumulate ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !dw) return e;  // no dw: the caller sums the partials later
    hipLaunchKernelGGL(sum_partials_split_kernel, dim3(grid_for(2 * C / 4, 16)), dim3(256), 0, s, dw, db,
                       (const float *)partial, P, C / 4, C / 4);
    return hipGetLastError();
}

hipError_t k_sum_partials_ld(float *dst, const float *src, int P, size_t n, size_t ld, bool accumulate,
                             hipStream_t s) {
    if (n % 4 || ld % 4 || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15) || P < 1) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        // src[p * ld + i], p < P, i < n
        audit(au, "sum_partials_kernel", "src", src, (long long)(P - 1) * (long long)ld + (long long)n, false);
        audit(au, "sum_partials_kernel", "dst", dst, (long long)n, true);
        return hipSuccess;
    }
    if (P >= 32)
        hipLaunchKernelGGL(sum_partials_wide_kernel, dim3(grid_for(n / 4, 16)), dim3(256), 0, s, dst, src, P, n / 4,
                           ld / 4, accumulate ? 1 : 0);
    else
        hipLaunchKernelGGL(sum_partials_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, s, dst, src, P, n / 4,
                           ld / 4, accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t k_sum_partials2(float *dst1, const float *src1, size_t n1, float *dst2, const float *src2, size_t n2, int P,
                          bool accumulate, hipStream_t s) {
    if (n1 % 4 || n2 % 4 || P < 1) return hipErrorInvalidValue;
    const uintptr_t al = (uintptr_t)dst1 | (uintptr_t)src1 | (uintptr_t)dst2 | (uintptr_t)src2;
    if (al & 15) return hipErrorInvalidValue;
    const size_t n = (n1 + n2) / 4;
    if (n == 0) return hipSuccess;
    if (AuditSink *au = audit_sink()) {
        audit(au, "sum_partials2_kernel", "src1", src1, (long long)P * (long long)n1, false);
        audit(au, "sum_partials2_kernel", "dst1", dst1, (long long)n1, true);
        audit(au, "sum_partials2_kernel", "src2", src2, (long long)P * (long long)n2, false);
        audit(au, "sum_partials2_kernel", "dst2", dst2, (long long)n2, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(sum_partials2_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, (floatx4 *)dst1,
                       (const floatx4 *)src1, n1 / 4, (floatx4 *)dst2, (const floatx4 *)src2, n2 / 4, P,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t k_sum_layers(float *dst1, const float *src1, size_t n1, float *dst2, const float *src2, size_t n2, int P,
                       int L, hipStream_t s) {
    if (n1 % 4 || n2 % 4 || P < 1 || L < 1) return hipErrorInvalidValue;
    const uintptr_t al = (uintptr_t)dst1 | (uintptr_t)src1 | (uintptr_t)dst2 | (uintptr_t)src2;
    if (al & 15) return hipErrorInvalidValue;
    const size_t n = (n1 + n2) / 4 * L;
    if (AuditSink *au = audit_sink()) {
        // layer l: dst + l n, src + l P n (P partials of n)
        audit(au, "sum_layers_kernel", "src1", src1, (long long)L * P * (long long)n1, false);
        audit(au, "sum_layers_kernel", "dst1", dst1, (long long)L * (long long)n1, true);
        audit(au, "sum_layers_kernel", "src2", src2, (long long)L * P * (long long)n2, false);
        audit(au, "sum_layers_kernel", "dst2", dst2, (long long)L * (long long)n2, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(sum_layers_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, (floatx4 *)dst1,
                       (const floatx4 *)src1, n1 / 4, (floatx4 *)dst2, (const floatx4 *)src2, n2 / 4, P, L);
    return hipGetLastError();
}

hipError_t k_sum_partials(float *dst, const float *src, int P, size_t n, bool accumulate, hipStream_t s) {
    return k_sum_partials_ld(dst, src, P, n, n, accumulate, s);
}

hipError_t k_attn_softmax_forward(float *att, long long nrows, int T, hipStream_t s) {
    if (T > 64 * SM_NV) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        audit(au, "attn_softmax_forward_kernel", "att", att, nrows * T, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(attn_softmax_forward_kernel, dim3(grid_for(nrows, 4)), dim3(256), 0, s, att, nrows, T);
    return hipGetLastError();
}

hipError_t k_attn_softmax_backward(float *dp, const float *att, long long nrows, int T, hipStream_t s) {
    if (T > 64 * SM_NV) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        audit(au, "attn_softmax_backward_kernel", "dp", dp, nrows * T, true);
        audit(au, "attn_softmax_backward_kernel", "att", att, nrows * T, false);
        return hipSuccess;
    }
    hipLaunchKernelGGL(attn_softmax_backward_kernel, dim3(grid_for(nrows, 4)), dim3(256), 0, s, dp, att, nrows, T);
    return hipGetLastError();
}

hipError_t k_crossentropy(float *logits, float *losses, const int32_t *tgt, int BT, int V, int Vp, float dscale,
                          const int32_t *gate, hipStream_t s) {
    if (Vp % 4) return hipErrorInvalidValue;
    const int n4 = Vp / 4;
    if (AuditSink *au = audit_sink()) {
        const char *k = k_crossentropy_name(Vp);
        audit(au, k, "logits", logits, (long long)BT * Vp, true);
        audit(au, k, "losses", losses, BT, true);
        audit(au, k, "tgt", tgt, BT, false);
        audit(au, k, "gate", gate, 1, false);
        return hipSuccess;
    }
    if (n4 <= 1024)
        hipLaunchKernelGGL(crossentropy_reg_kernel<1>, dim3(BT), dim3(1024), 0, s, logits, losses, tgt, V, Vp, dscale, gate);
    else if (n4 <= 4 * 1024)
        hipLaunchKernelGGL(crossentropy_reg_kernel<4>, dim3(BT), dim3(1024), 0, s, logits, losses, tgt, V, Vp, dscale, gate);
    else if (n4 <= 13 * 1024)
        hipLaunchKernelGGL(crossentropy_reg_kernel<13>, dim3(BT), dim3(1024), 0, s, logits, losses, tgt, V, Vp, dscale, gate);
    else
        hipLaunchKernelGGL(crossentropy_kernel, dim3(BT), dim3(256), 0, s, logits, losses, tgt, V, Vp, dscale, gate);
    return hipGetLastError();
}

const char *k_crossentropy_name(int Vp) {
    const int n4 = Vp / 4;
    if (n4 <= 1024) return "crossentropy_reg_kernel<1>";
    if (n4 <= 4 * 1024) return "crossentropy_reg_kernel<4>";
    if (n4 <= 13 * 1024) return "crossentropy_reg_kernel<13>";
    return "crossentropy_kernel";
}

hipError_t k_mean(float *loss, const float *losses, int n, hipStream_t s) {
    if (AuditSink *au = audit_sink()) {
        audit(au, "mean_kernel", "losses", losses, n, false);
        audit(au, "mean_kernel", "loss", loss, 1, true);
        return hipSuccess;
    }
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, s, loss, losses, n);
    return hipGetLastError();
}

hipError_t k_gelu_forward(float *out, const float *inp, size_t n, hipStream_t s) {
    if (n % 4) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        audit(au, "gelu_forward_kernel", "out", out, (long long)n, true);
        audit(au, "gelu_forward_kernel", "inp", inp, (long long)n, false);
        return hipSuccess;
    }
    hipLaunchKernelGGL(gelu_forward_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, s, (floatx4 *)out,
                       (const floatx4 *)inp, n / 4);
    return hipGetLastError();
}

hipError_t k_gelu_backward(float *dinp, const float *inp, const float *dout, size_t n, hipStream_t s) {
    if (n % 4) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        audit(au, "gelu_backward_kernel", "dinp", dinp, (long long)n, true);
        audit(au, "gelu_backward_kernel", "inp", inp, (long long)n, false);
        audit(au, "gelu_backward_kernel", "dout", dout, (long long)n, false);
        return hipSuccess;
    }
    hipLaunchKernelGGL(gelu_backward_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, s, (floatx4 *)dinp,
                       (const floatx4 *)inp, (const floatx4 *)dout, n / 4);
    return hipGetLastError();
}

hipError_t k_adamw(float *params, const float *grads, float *m, float *v, size_t n, float lr, float b1, float b2,
                   float eps, float wd, float c1, float c2, const int32_t *gate, hipStream_t s) {
    if (n % 4) return hipErrorInvalidValue;
    size_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    const size_t g = (n4 + 256 * ADAMW_U - 1) / (256 * ADAMW_U);
    if (g > 0x7fffffff) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        audit(au, "adamw_kernel", "params", params, (long long)n, true);
        audit(au, "adamw_kernel", "grads", grads, (long long)n, false);
        audit(au, "adamw_kernel", "m", m, (long long)n, true);
        audit(au, "adamw_kernel", "v", v, (long long)n, true);
        audit(au, "adamw_kernel", "gate", gate, 1, false);
        return hipSuccess;
    }
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)g), dim3(256), 0, s, (floatx4 *)params, (const floatx4 *)grads,
                       (floatx4 *)m, (floatx4 *)v, n4, lr, b1, b2, eps, wd, 1.0f / c1, 1.0f / c2, gate);
    return hipGetLastError();
}
