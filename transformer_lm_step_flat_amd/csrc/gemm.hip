// fp32 MFMA GEMM for gfx950.  See gemm.h for the contract.
//
// One workgroup = 4 wavefronts (2 x 2) computes a BM x BN tile of C; each
// wavefront owns a (BM/2) x (BN/2) sub-tile made of 32 x 32 MFMA blocks with
// the accumulators held in registers.  The K loop stages BK = 32 or 64 slices
// of A and B through LDS: while the MFMAs consume the current slice, the next one
// is already on its way from global memory into registers.
//
// K-index assignment inside a slice: v_mfma_f32_32x32x2_f32 takes two k
// values per instruction, one from each half of the wavefront (lanes 0-31
// and 32-63).  Lane half h feeds k = h*BK/2 + j for the j-th instruction of
// the slice, so each lane walks BK/2 consecutive k: for a K-contiguous operand
// that is BK/8 16-byte LDS reads per 32 x 32 block per slice.  Any pairing of k to
// instruction slots gives the same sum, so this only changes rounding order.
//
// LDS layouts: a K-contiguous operand is kept [mn][k] with a row pitch of
// BK + 4 floats (16-byte reads by 8 consecutive lanes hit all 32 banks once);
// an MN-contiguous operand is kept [k][mn] and read one float per lane along
// mn (32 consecutive words per half-wave).
#include "common.h"
#include "audit.h"
#include "gemm.h"

namespace {

constexpr int GEMM_THREADS = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Two 4-float fragments (8 consecutive k) rounded to bfloat16, to nearest
// even (v_cvt_pk_bf16_f32), as one operand of v_mfma_f32_32x32x16_bf16.
__device__ __forceinline__ bf16x8 to_bf16x8(const floatx4 &lo, const floatx4 &hi) {
    const bf16x8 r = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                      (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
    return r;
}

// An epilogue mode as a type, so that one epilogue body serves every mode
template <int V>
struct EpiTag {
    static constexpr int value = V;
};

struct GemmArgs {
    const float *A, *B;
    float *C, *C2;
    const float *bias, *aux;
    float *colsum;
    long long lda, ldb, ldc, ldaux;
    long long sAo, sAi, sBo, sBi, sCo, sCi, sCs;
    float alpha;
    int M, N, K;
    int epi, causal;
    int nbi, ksplit, kchunk;
    int tiles_m, tiles_n, group_m;
};

// Workgroups are handed to the 8 XCDs round-robin by id.  Renumber so that
// each XCD works on one contiguous run of tiles (which then share operand
// tiles in that XCD's L2).  The map is a bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int X = 8;
    int q = n / X, r = n % X;
    int x = bid % X, loc = bid / X;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + loc;
}

// Tile order: groups of `g` tile-rows walked column by column.
__device__ __forceinline__ void group_order(int bid, int tiles_m, int tiles_n, int g, int &tm, int &tn) {
    int width = g * tiles_n;
    int grp = bid / width;
    int first = grp * g;
    int gs = min(tiles_m - first, g);
    int r = bid - grp * width;
    tm = first + r % gs;
    tn = r / gs;
}

// LDS floats of the two operand tiles
template <int BM, int BN, bool AK, bool BKC, int BK>
struct TileLds {
    static constexpr int KP = BK + 4;  // pitch of a K-contiguous LDS tile
    static constexpr int A = AK ? BM * KP : BK * BM;
    static constexpr int B = BKC ? BN * KP : BK * BN;
};

// One BM x BN output tile (row tile tm, column tile tn), batch / split
// index z, operand tiles staged in As / Bs.  kr0 >= 0 replaces the tile's K
// range by [kr0, kr1).  FULL: the launch guarantees that every tile lies
// inside M x N and every K range is a whole number of BK slices (no bounds
// tests anywhere in the K loop).  PREC 0: fp32 products
// (v_mfma_f32_32x32x2_f32); PREC 1: the operands are rounded to bfloat16 as
// they leave LDS and multiplied with v_mfma_f32_32x32x16_bf16 (fp32
// accumulation; memory, LDS and epilogue stay fp32).
template <int BM, int BN, bool AK, bool BKC, int BK, bool FULL = false, int PREC = 0>
__device__ __forceinline__ void gemm_tile(const GemmArgs &p, int tm, int tn, int z, float *__restrict__ As,
                                          float *__restrict__ Bs, int kr0 = -1, int kr1 = 0) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int KP = TileLds<BM, BN, AK, BKC, BK>::KP;
    constexpr int A_F4 = BM * BK / 4 / GEMM_THREADS;
    constexpr int B_F4 = BN * BK / 4 / GEMM_THREADS;
    static_assert(A_F4 >= 1 && B_F4 >= 1, "tile too small for 256 threads");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, h = lane >> 5;

    const int s = z % p.ksplit, zb = z / p.ksplit;
    const int zo = zb / p.nbi, zi = zb % p.nbi;
    const float *__restrict__ A = p.A + zo * p.sAo + zi * p.sAi;
    const float *__restrict__ B = p.B + zo * p.sBo + zi * p.sBi;
    float *__restrict__ C = p.C + zo * p.sCo + zi * p.sCi + s * p.sCs;

    const int m0 = tm * BM, n0 = tn * BN;
    if (p.causal == CAUSAL_SKIP_UPPER && n0 >= m0 + BM) return;
    int kbeg = s * p.kchunk, kend = min(p.K, kbeg + p.kchunk);
    if (p.causal == CAUSAL_KEND) kend = min(kend, m0 + BM);
    if (p.causal == CAUSAL_KSTART) kbeg = max(kbeg, m0);
    if (kr0 >= 0) {
        kbeg = kr0;
        kend = kr1;
    }

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
        for (int j = 0; j < NI; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    floatx4 ra[A_F4], rb[B_F4];
    const int M = p.M, N = p.N;
    // Column sums of A (only MN-contiguous A, only the first tile column),
    // accumulated from the A values each thread loads: for an MN-contiguous
    // A a thread's 16-byte loads always cover the same 4 columns.
    const bool do_colsum = !AK && p.colsum != nullptr && tn == 0;
    floatx4 csum = {0.f, 0.f, 0.f, 0.f};
    const long long lda = p.lda, ldb = p.ldb;

    // Whole-slice loads of a tile inside M x N.  Where GEMM_THREADS is a
    // multiple of the float4s per row of the staged layout (BK / 4 for a
    // K-contiguous operand, BM / 4 or BN / 4 otherwise), thread tid's float4
    // number i (f = tid + 256 i) sits at
    // a per-thread address plus an offset common to the workgroup, so one
    // pointer per operand and thread can serve every load.  That form is
    // used when B is MN-contiguous (the weight- and input-gradient products);
    // with both operands K-contiguous (the forward products) an address per
    // load measured faster (fc forward -3 %; the gradient pairs +1 to 8 %
    // the other way round).
    constexpr bool kEvenA = !BKC && GEMM_THREADS % (AK ? BK / 4 : BM / 4) == 0;
    constexpr bool kEvenB = !BKC && GEMM_THREADS % (BN / 4) == 0;
    // The per-thread part of that address is a 32-bit byte offset (the same
    // for every slice and load), the rest a scalar base (tile origin, slice
    // and load index): the loads then take no vector instructions for their
    // addresses, which would take issue cycles from the matrix unit.
    const unsigned va = (unsigned)(4 * (AK ? (long long)(tid / (BK / 4)) * lda + 4 * (tid % (BK / 4))
                                           : (long long)(tid / (BM / 4)) * lda + 4 * (tid % (BM / 4))));
    const unsigned vb = (unsigned)(4 * (BKC ? (long long)(tid / (BK / 4)) * ldb + 4 * (tid % (BK / 4))
                                            : (long long)(tid / (BN / 4)) * ldb + 4 * (tid % (BN / 4))));
    const char *const a0 = (const char *)(AK ? A + (long long)m0 * lda : A + m0);
    const char *const b0 = (const char *)(BKC ? B + (long long)n0 * ldb : B + n0);
    // (buffer loads: a resource per slice whose base is the slice origin, a
    // scalar offset per load, the thread's offset; all offsets stay small)
    auto fast_load = [&](int k0) {
        const auto ar = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a0 + 4 * (AK ? (long long)k0 : (long long)k0 * lda)), (short)0, -1, 0x00020000);
        const auto br = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(b0 + 4 * (BKC ? (long long)k0 : (long long)k0 * ldb)), (short)0, -1, 0x00020000);
#pragma unroll
        for (int i = 0; i < A_F4; i++) {
            if constexpr (kEvenA) {
                const int so = (int)(4 * (long long)(GEMM_THREADS / (AK ? BK / 4 : BM / 4)) * i * lda);
                ra[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(ar, va, so, 0));
            } else {
                const int f = tid + GEMM_THREADS * i;
                const int gm = AK ? m0 + f / (BK / 4) : m0 + 4 * (f % (BM / 4));
                const int gk = AK ? k0 + 4 * (f % (BK / 4)) : k0 + f / (BM / 4);
                ra[i] = *(const floatx4 *)(AK ? A + gm * lda + gk : A + gk * lda + gm);
            }
        }
#pragma unroll
        for (int i = 0; i < B_F4; i++) {
            if constexpr (kEvenB) {
                const int so = (int)(4 * (long long)(GEMM_THREADS / (BKC ? BK / 4 : BN / 4)) * i * ldb);
                rb[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(br, vb, so, 0));
            } else {
                const int f = tid + GEMM_THREADS * i;
                const int gn = BKC ? n0 + f / (BK / 4) : n0 + 4 * (f % (BN / 4));
                const int gk = BKC ? k0 + 4 * (f % (BK / 4)) : k0 + f / (BN / 4);
                rb[i] = *(const floatx4 *)(BKC ? B + gn * ldb + gk : B + gk * ldb + gn);
            }
        }
    };
    // A tile inside M x N whose slice lies inside [kbeg, kend) loads without
    // bounds tests: no predication, no zeroing of the load targets.  Vector
    // ALU and global-memory instructions do not issue on a SIMD while another
    // wavefront there keeps its matrix unit busy, so every such instruction
    // saved shortens the K loop (measured: -1.5 % step time).
    const bool interior = m0 + BM <= M && n0 + BN <= N;
    auto gload = [&](int k0) {
        if (interior && k0 + BK <= kend) {
            fast_load(k0);
            return;
        }
#pragma unroll
        for (int i = 0; i < A_F4; i++) {
            int f = tid + GEMM_THREADS * i;
            int gm, gk;
            if (AK) { gm = m0 + f / (BK / 4); gk = k0 + 4 * (f % (BK / 4)); }
            else    { gk = k0 + f / (BM / 4); gm = m0 + 4 * (f % (BM / 4)); }
            if (gm < M && gk < kend)
                ra[i] = *(const floatx4 *)(AK ? A + gm * lda + gk : A + gk * lda + gm);
            else
                ra[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < B_F4; i++) {
            int f = tid + GEMM_THREADS * i;
            int gn, gk;
            if (BKC) { gn = n0 + f / (BK / 4); gk = k0 + 4 * (f % (BK / 4)); }
            else     { gk = k0 + f / (BN / 4); gn = n0 + 4 * (f % (BN / 4)); }
            if (gn < N && gk < kend)
                rb[i] = *(const floatx4 *)(BKC ? B + gn * ldb + gk : B + gk * ldb + gn);
            else
                rb[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto lstore = [&]() {
        // (a scalar condition: the sums are skipped, not computed and discarded,
        // by the tiles that do not keep them)
        if (!AK && __builtin_amdgcn_readfirstlane((int)do_colsum)) {
#pragma unroll
            for (int i = 0; i < A_F4; i++) csum += ra[i];
        }
#pragma unroll
        for (int i = 0; i < A_F4; i++) {
            int f = tid + GEMM_THREADS * i;
            if (AK) *(floatx4 *)&As[(f / (BK / 4)) * KP + 4 * (f % (BK / 4))] = ra[i];
            else    *(floatx4 *)&As[(f / (BM / 4)) * BM + 4 * (f % (BM / 4))] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_F4; i++) {
            int f = tid + GEMM_THREADS * i;
            if (BKC) *(floatx4 *)&Bs[(f / (BK / 4)) * KP + 4 * (f % (BK / 4))] = rb[i];
            else     *(floatx4 *)&Bs[(f / (BN / 4)) * BN + 4 * (f % (BN / 4))] = rb[i];
        }
    };

    // The fragment of 4 consecutive k (h * BK / 2 + 4 q ..) of row block i of
    // A and column block j of B that this lane feeds to the matrix unit.
    auto frag_a = [&](int i, int q) {
        const int mm = wm * WM + i * 32 + l32;
        floatx4 a;
        if (AK) {
            a = *(const floatx4 *)&As[mm * KP + h * (BK / 2) + 4 * q];
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++) a[e] = As[(h * (BK / 2) + 4 * q + e) * BM + mm];
        }
        return a;
    };
    auto frag_b = [&](int j, int q) {
        const int nn = wn * WN + j * 32 + l32;
        floatx4 b;
        if (BKC) {
            b = *(const floatx4 *)&Bs[nn * KP + h * (BK / 2) + 4 * q];
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++) b[e] = Bs[(h * (BK / 2) + 4 * q + e) * BN + nn];
        }
        return b;
    };
    // The MFMAs of the slice in LDS.  fp32: one 32x32x2 per k pair (lane half
    // h giving one k of the pair); bf16: one 32x32x16 per 8 consecutive k of
    // each lane half (fragments q and q + 1).
    auto slice_mfma = [&]() {
        if constexpr (PREC == 0) {
#pragma unroll
            for (int q = 0; q < BK / 8; q++) {
                floatx4 a[MI], b[NI];
#pragma unroll
                for (int i = 0; i < MI; i++) a[i] = frag_a(i, q);
#pragma unroll
                for (int j = 0; j < NI; j++) b[j] = frag_b(j, q);
#pragma unroll
                for (int e = 0; e < 4; e++)
#pragma unroll
                    for (int i = 0; i < MI; i++)
#pragma unroll
                        for (int j = 0; j < NI; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
            }
        } else {
            static_assert(BK % 16 == 0, "bf16 slices take 8 k per lane half");
#pragma unroll
            for (int q2 = 0; q2 < BK / 16; q2++) {
                bf16x8 a[MI], b[NI];
#pragma unroll
                for (int i = 0; i < MI; i++) a[i] = to_bf16x8(frag_a(i, 2 * q2), frag_a(i, 2 * q2 + 1));
#pragma unroll
                for (int j = 0; j < NI; j++) b[j] = to_bf16x8(frag_b(j, 2 * q2), frag_b(j, 2 * q2 + 1));
#pragma unroll
                for (int i = 0; i < MI; i++)
#pragma unroll
                    for (int j = 0; j < NI; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    if constexpr (FULL) {
        // one slice's MFMAs (the wave priority is raised around them, as in
        // the general loop below)
        auto mfma_slice = [&]() { slice_mfma(); };

        // Every slice is full: a branch-free loop, the last slice peeled off.
        // The next slice's loads are placed one after each of the first
        // MFMAs, so that they issue while this wavefront's own MFMAs run
        // instead of waiting behind those of other workgroups.
        int k0 = kbeg;
        if (kbeg < kend) fast_load(kbeg);
        for (; k0 + BK < kend; k0 += BK) {
            __syncthreads();
            lstore();
            __syncthreads();
            __builtin_amdgcn_s_setprio(1);
            fast_load(k0 + BK);
            mfma_slice();
            constexpr int NMFMA = MI * NI * (PREC == 0 ? BK / 2 : BK / 16);
            constexpr int NPAIR = NMFMA < A_F4 + B_F4 ? NMFMA : A_F4 + B_F4;
#pragma unroll
            for (int i = 0; i < NPAIR; i++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if (k0 < kend) {
            __syncthreads();
            lstore();
            __syncthreads();
            __builtin_amdgcn_s_setprio(1);
            mfma_slice();
            __builtin_amdgcn_s_setprio(0);
        }
    } else {
        if (kbeg < kend) gload(kbeg);
        for (int k0 = kbeg; k0 < kend; k0 += BK) {
            __syncthreads();
            lstore();
            __syncthreads();
            if (k0 + BK < kend) gload(k0 + BK);
            // Raised wave priority while this slice's MFMAs issue: the sequencer
            // then prefers the wavefronts feeding the matrix unit over those of
            // other workgroups that are storing their next slice to LDS or
            // waiting at a barrier (measured: without it the step takes 3 %
            // longer; raising the load phase's priority instead costs 3 to 4 %).
            __builtin_amdgcn_s_setprio(1);
            slice_mfma();
            __builtin_amdgcn_s_setprio(0);
        }
    }

    if (!AK && do_colsum) {
        // combine the partial sums of the threads sharing 4 columns, in a fixed order
        constexpr int CQ = BM / 4, RL = GEMM_THREADS / CQ;
        __syncthreads();
        *(floatx4 *)&As[4 * tid] = csum;
        __syncthreads();
        if (tid < CQ && m0 + 4 * tid < M) {
            floatx4 t = *(const floatx4 *)&As[4 * tid];
#pragma unroll
            for (int g = 1; g < RL; g++) t += *(const floatx4 *)&As[4 * (g * CQ + tid)];
            float *dst = p.ksplit > 1 ? p.colsum + (long long)s * M + m0 + 4 * tid : p.colsum + m0 + 4 * tid;
#pragma unroll
            for (int e = 0; e < 4; e++) dst[e] = p.ksplit > 1 ? t[e] : dst[e] + t[e];
        }
    }

    // Epilogue.  32x32 accumulator layout: lane l holds column l % 32 and
    // rows 8*(r/4) + 4*(l/32) + r%4 for its registers r = 0..15.  Operands
    // that live in memory (C for accumulation, the residual or the GELU
    // input) are loaded for a whole 32 x 32 block before any arithmetic, so
    // that their latencies overlap.
    // The mode is dispatched once, outside the element loops; each mode's loop
    // has no per-element branching on it.  Whole tiles (FULL) skip the bounds
    // tests, and a row's address is the block's row base plus a multiple of ldc.
    auto epilogue = [&](auto tag) {
        constexpr int EPI = decltype(tag)::value;
        constexpr bool gather = EPI == EPI_ACCUM || EPI == EPI_RESID || EPI == EPI_GELU_BWD;
        const float *src = EPI == EPI_ACCUM ? C : p.aux;
        const long long lds_ = EPI == EPI_ACCUM ? p.ldc : p.ldaux;
        const long long ldc = p.ldc;
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
            for (int j = 0; j < NI; j++) {
                const int n = n0 + wn * WN + j * 32 + l32;
                if (!FULL && n >= N) continue;
                const int mb = m0 + wm * WM + i * 32 + h * 4;  // row of register 0
                float ext[16];
                if constexpr (gather) {
                    const float *sb = src + (long long)mb * lds_ + n;
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int dr = (r >> 2) * 8 + (r & 3);
                        ext[r] = (FULL || mb + dr < M) ? sb[dr * lds_] : 0.0f;
                    }
                }
                const float bn = p.bias ? p.bias[n] : 0.0f;
                float *cb = C + (long long)mb * ldc + n;
                float *c2b = EPI == EPI_GELU ? p.C2 + (long long)mb * ldc + n : nullptr;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int dr = (r >> 2) * 8 + (r & 3);
                    if (!FULL && mb + dr >= M) continue;
                    const float v = p.alpha * acc[i][j][r];
                    const long long off = dr * ldc;
                    if constexpr (EPI == EPI_STORE) cb[off] = v + bn;
                    if constexpr (EPI == EPI_ACCUM) cb[off] = ext[r] + v;
                    if constexpr (EPI == EPI_RESID) cb[off] = v + bn + ext[r];
                    if constexpr (EPI == EPI_GELU) {
                        const float pre = v + bn;
                        cb[off] = pre;
                        c2b[off] = gelu_fwd(pre);
                    }
                    if constexpr (EPI == EPI_GELU_BWD) cb[off] = v * gelu_grad(ext[r]);
                }
            }
    };
    switch (p.epi) {
        case EPI_STORE: epilogue(EpiTag<EPI_STORE>{}); break;
        case EPI_ACCUM: epilogue(EpiTag<EPI_ACCUM>{}); break;
        case EPI_RESID: epilogue(EpiTag<EPI_RESID>{}); break;
        case EPI_GELU: epilogue(EpiTag<EPI_GELU>{}); break;
        case EPI_GELU_BWD: epilogue(EpiTag<EPI_GELU_BWD>{}); break;
    }
}

template <int BM, int BN, bool AK, bool BKC, int BK, int LB, bool FULL>
__global__ __launch_bounds__(GEMM_THREADS, LB) void gemm_kernel(GemmArgs p) {
    using L = TileLds<BM, BN, AK, BKC, BK>;
    __shared__ __attribute__((aligned(16))) float As[L::A];
    __shared__ __attribute__((aligned(16))) float Bs[L::B];
    int tm, tn;
    group_order(xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n), p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    gemm_tile<BM, BN, AK, BKC, BK, FULL>(p, tm, tn, blockIdx.z, As, Bs);
}

// The same with bfloat16 products (PREC 1 of gemm_tile).
template <int BM, int BN, bool AK, bool BKC, int BK, int LB, bool FULL>
__global__ __launch_bounds__(GEMM_THREADS, LB) void gemm_bf16_kernel(GemmArgs p) {
    using L = TileLds<BM, BN, AK, BKC, BK>;
    __shared__ __attribute__((aligned(16))) float As[L::A];
    __shared__ __attribute__((aligned(16))) float Bs[L::B];
    int tm, tn;
    group_order(xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n), p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    gemm_tile<BM, BN, AK, BKC, BK, FULL, 1>(p, tm, tn, blockIdx.z, As, Bs);
}

// Causal products whose K range grows (KEND) or shrinks (KSTART) with the row
// tile: a workgroup takes row tiles i and tiles_m - 1 - i of one column, whose
// K ranges add up to the same length for every workgroup.
template <int BM, int BN, bool AK, bool BKC, int BK, int LB>
__global__ __launch_bounds__(GEMM_THREADS, LB) void gemm_fold_kernel(GemmArgs p) {
    using L = TileLds<BM, BN, AK, BKC, BK>;
    __shared__ __attribute__((aligned(16))) float As[L::A];
    __shared__ __attribute__((aligned(16))) float Bs[L::B];
    const int half = (p.tiles_m + 1) / 2;
    const int t = xcd_remap(blockIdx.x, half * p.tiles_n);
    const int tn = t / half, i = t % half, j = p.tiles_m - 1 - i;
    const int npass = i == j ? 1 : 2;
    for (int pass = 0; pass < npass; pass++)
        gemm_tile<BM, BN, AK, BKC, BK>(p, pass == 0 ? j : i, tn, blockIdx.z, As, Bs);
}

// The folded causal product (KEND) with twice the workgroups: the pair of
// row tiles (i, j = tiles_m - 1 - i) has kj + ki k values in all (one tile if
// i == j); workgroup s = 0 takes the first half of row tile j's range into C,
// s = 1 the rest of j's range into pp (a compact copy of C's layout: the
// partial sums) and all of row tile i into C.  fold_split_sum_kernel then
// adds the partials into the row tiles j >= tiles_m / 2.  Same result as one
// workgroup per pair up to the order of two partial sums; twice the
// workgroups for products with few row tiles.  FULL: whole tiles and K a
// whole number of slices (every range above is then whole slices too).
template <int BM, int BN, bool AK, bool BKC, int BK, int LB, bool FULL>
__global__ __launch_bounds__(GEMM_THREADS, LB) void gemm_fold_split_kernel(GemmArgs p, GemmArgs pp) {
    using L = TileLds<BM, BN, AK, BKC, BK>;
    __shared__ __attribute__((aligned(16))) float As[L::A];
    __shared__ __attribute__((aligned(16))) float Bs[L::B];
    const int half = (p.tiles_m + 1) / 2;
    const int t = xcd_remap(blockIdx.x, 2 * half * p.tiles_n);
    const int s = t & 1, u = t >> 1;
    const int tn = u / half, i = u % half, j = p.tiles_m - 1 - i;
    const int kj = min(p.K, (j + 1) * BM), ki = min(p.K, (i + 1) * BM);
    const int tot = i == j ? kj : kj + ki;
    const int hk = min(kj, (tot / 2 + BK - 1) / BK * BK);
    if (s == 0) {
        gemm_tile<BM, BN, AK, BKC, BK, FULL>(p, j, tn, blockIdx.z, As, Bs, 0, hk);
    } else {
        gemm_tile<BM, BN, AK, BKC, BK, FULL>(pp, j, tn, blockIdx.z, As, Bs, hk, kj);
        if (i != j) gemm_tile<BM, BN, AK, BKC, BK, FULL>(p, i, tn, blockIdx.z, As, Bs, 0, ki);
    }
}

// C(z, m, n) += part[z][m][n] for the rows m >= m0 of every batch z; one
// thread per 4 columns.
__global__ __launch_bounds__(256) void fold_split_sum_kernel(float *C, long long ldc, long long sCo, long long sCi,
                                                             int nbi, const float *part, int M, int N, int m0,
                                                             long long n4) {
    const long long f = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (f >= n4) return;
    const int N4 = N / 4, R = M - m0;
    const int c4 = (int)(f % N4);
    const long long r = f / N4;
    const int m = m0 + (int)(r % R);
    const int z = (int)(r / R);
    const int zo = z / nbi, zi = z % nbi;
    float *c = C + zo * sCo + zi * sCi + (long long)m * ldc + 4 * c4;
    const floatx4 a = *(const floatx4 *)c;
    const floatx4 b = *(const floatx4 *)(part + ((long long)z * M + m) * N + 4 * c4);
    *(floatx4 *)c = a + b;
}

// Two independent products in one grid of w = w1 + w2 workgroups (w1 of
// problem 1: its tiles, then its batches / splits; w2 of problem 2).  Both
// use the same tile shape.  Each XCD gets an eighth of each problem, as one
// contiguous run of problem 1 followed by one of problem 2, so that the work
// per XCD is balanced and operand tiles are shared within an XCD's L2.
template <int BM, int BN, int BK, bool AK1, bool BKC1, bool AK2, bool BKC2, bool FULL, int PREC>
__device__ __forceinline__ void pair_body(const GemmArgs &p1, const GemmArgs &p2, int w1, int w) {
    using L1 = TileLds<BM, BN, AK1, BKC1, BK>;
    using L2 = TileLds<BM, BN, AK2, BKC2, BK>;
    __shared__ __attribute__((aligned(16))) float As[L1::A > L2::A ? L1::A : L2::A];
    __shared__ __attribute__((aligned(16))) float Bs[L1::B > L2::B ? L1::B : L2::B];
    const int X = 8;
    const int x = blockIdx.x % X, j = blockIdx.x / X;  // XCD, and order within it
    const int q1 = w1 / X, m1 = w1 % X;
    const int r1 = q1 + (x < m1);                    // problem-1 workgroups of this XCD
    const int s1 = x * q1 + min(x, m1);              // their first index
    if (j < r1) {
        const int g = s1 + j, nt = p1.tiles_m * p1.tiles_n;
        int tm, tn;
        group_order(g % nt, p1.tiles_m, p1.tiles_n, p1.group_m, tm, tn);
        gemm_tile<BM, BN, AK1, BKC1, BK, FULL, PREC>(p1, tm, tn, g / nt, As, Bs);
    } else {
        const int s2 = x * (w / X) + min(x, w % X) - s1;  // workgroups of XCDs before x, less problem 1's
        const int g = s2 + j - r1, nt = p2.tiles_m * p2.tiles_n;
        int tm, tn;
        group_order(g % nt, p2.tiles_m, p2.tiles_n, p2.group_m, tm, tn);
        gemm_tile<BM, BN, AK2, BKC2, BK, FULL, PREC>(p2, tm, tn, g / nt, As, Bs);
    }
}

template <int BM, int BN, int BK, int LB, bool AK1, bool BKC1, bool AK2, bool BKC2, bool FULL>
__global__ __launch_bounds__(GEMM_THREADS, LB) void gemm_pair_kernel(GemmArgs p1, GemmArgs p2, int w1, int w) {
    pair_body<BM, BN, BK, AK1, BKC1, AK2, BKC2, FULL, 0>(p1, p2, w1, w);
}

// The same with bfloat16 products.
template <int BM, int BN, int BK, int LB, bool AK1, bool BKC1, bool AK2, bool BKC2, bool FULL>
__global__ __launch_bounds__(GEMM_THREADS, LB) void gemm_pair_bf16_kernel(GemmArgs p1, GemmArgs p2, int w1, int w) {
    pair_body<BM, BN, BK, AK1, BKC1, AK2, BKC2, FULL, 1>(p1, p2, w1, w);
}

// Tile grid and the K range of each split (a whole number of BK slices).
template <int BM, int BN, int BK>
void set_tiles(const GemmDesc &d, GemmArgs &a) {
    a.tiles_m = (d.M + BM - 1) / BM;
    a.tiles_n = (d.N + BN - 1) / BN;
    a.group_m = 8;
    const int kc = (d.K + d.ksplit - 1) / d.ksplit;
    a.kchunk = kc > 0 ? (kc + BK - 1) / BK * BK : BK;
}

// Whether every tile of d lies inside M x N and every K range (one per
// split) is a whole number of BK slices: the launch may then use the
// kernels without bounds tests.  Causal products are excluded.
bool gemm_full(const GemmDesc &d, int bm, int bn, int bk) {
    return d.causal == 0 && d.M % bm == 0 && d.N % bn == 0 && d.K % bk == 0;
}
// the folded causal product's ranges are whole slices when its tiles are whole
// and K is whole slices (row-tile ends are multiples of bm, itself of bk)
bool fold_split_full(const GemmDesc &d, int bm, int bn, int bk) {
    return d.M % bm == 0 && d.N % bn == 0 && d.K % bk == 0 && bm % bk == 0;
}

template <int BM, int BN, bool AKV, bool BKV, int BK, int LB>
void launch_gemm_kernel(bool full, int prec, dim3 grid, hipStream_t stream, const GemmArgs &a) {
    if (prec == 0) {
        if (full)
            hipLaunchKernelGGL((gemm_kernel<BM, BN, AKV, BKV, BK, LB, true>), grid, dim3(GEMM_THREADS), 0, stream, a);
        else
            hipLaunchKernelGGL((gemm_kernel<BM, BN, AKV, BKV, BK, LB, false>), grid, dim3(GEMM_THREADS), 0, stream, a);
    } else {
        if (full)
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AKV, BKV, BK, LB, true>), grid, dim3(GEMM_THREADS), 0, stream,
                               a);
        else
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AKV, BKV, BK, LB, false>), grid, dim3(GEMM_THREADS), 0, stream,
                               a);
    }
}

template <int BM, int BN, int BK, int LB>
hipError_t launch_tile(const GemmDesc &d, const GemmArgs &a0, hipStream_t stream) {
    GemmArgs a = a0;
    set_tiles<BM, BN, BK>(d, a);
    long long nb = (long long)d.nbo * d.nbi * d.ksplit;
    if (nb > 65535) return hipErrorInvalidValue;
    if (d.part && d.causal == CAUSAL_KEND && a.tiles_m > 1) {
        const int half = (a.tiles_m + 1) / 2;
        GemmArgs pp = a;
        pp.C = d.part;
        pp.ldc = d.N;
        pp.sCi = (long long)d.M * d.N;
        pp.sCo = pp.sCi * d.nbi;
        dim3 g(2 * half * a.tiles_n, 1, (unsigned)nb);
        if (!d.a_kcontig || d.b_kcontig) return hipErrorInvalidValue;
        if (fold_split_full(d, BM, BN, BK))
            hipLaunchKernelGGL((gemm_fold_split_kernel<BM, BN, true, false, BK, LB, true>), g, dim3(GEMM_THREADS), 0,
                               stream, a, pp);
        else
            hipLaunchKernelGGL((gemm_fold_split_kernel<BM, BN, true, false, BK, LB, false>), g, dim3(GEMM_THREADS), 0,
                               stream, a, pp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int m0 = a.tiles_m / 2 * BM;
        const long long n4 = nb * (long long)(d.M - m0) * (d.N / 4);
        hipLaunchKernelGGL(fold_split_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, d.C, d.ldc,
                           d.sCo, d.sCi, d.nbi, (const float *)d.part, d.M, d.N, m0, n4);
        return hipGetLastError();
    }
    if ((d.causal == CAUSAL_KEND || d.causal == CAUSAL_KSTART) && a.tiles_m > 1) {
        dim3 g((a.tiles_m + 1) / 2 * a.tiles_n, 1, (unsigned)nb);
        if (d.a_kcontig && !d.b_kcontig)
            hipLaunchKernelGGL((gemm_fold_kernel<BM, BN, true, false, BK, LB>), g, dim3(GEMM_THREADS), 0, stream, a);
        else if (!d.a_kcontig && !d.b_kcontig)
            hipLaunchKernelGGL((gemm_fold_kernel<BM, BN, false, false, BK, LB>), g, dim3(GEMM_THREADS), 0, stream, a);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    dim3 grid(a.tiles_m * a.tiles_n, 1, (unsigned)nb);
    const bool full = gemm_full(d, BM, BN, BK);
    if (d.a_kcontig && d.b_kcontig)
        launch_gemm_kernel<BM, BN, true, true, BK, LB>(full, d.prec, grid, stream, a);
    else if (d.a_kcontig && !d.b_kcontig)
        launch_gemm_kernel<BM, BN, true, false, BK, LB>(full, d.prec, grid, stream, a);
    else if (!d.a_kcontig && !d.b_kcontig)
        launch_gemm_kernel<BM, BN, false, false, BK, LB>(full, d.prec, grid, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// The paired kernel for whole tiles is used for the 128 x 128 and 64 x 64
// shapes; at 128 x 64 it measured slower than the general one (fc and
// attproj backward: +7 % and +42 %), so that shape keeps the general kernel.
template <int BM, int BN>
constexpr bool pair_full_shape() {
    return true;
}

template <int BM, int BN, int BK, int LB>
hipError_t launch_pair(const GemmDesc &d1, const GemmArgs &a1_, const GemmDesc &d2, const GemmArgs &a2_,
                       hipStream_t stream) {
    GemmArgs a1 = a1_, a2 = a2_;
    set_tiles<BM, BN, BK>(d1, a1);
    set_tiles<BM, BN, BK>(d2, a2);
    const long long w1 = (long long)a1.tiles_m * a1.tiles_n * d1.nbo * d1.nbi * d1.ksplit;
    const long long w2 = (long long)a2.tiles_m * a2.tiles_n * d2.nbo * d2.nbi * d2.ksplit;
    if (w1 + w2 > (1LL << 30)) return hipErrorInvalidValue;
    // the one instantiation used: a weight gradient (both MN-contiguous) beside an input gradient
    if (d1.a_kcontig || d1.b_kcontig || !d2.a_kcontig || d2.b_kcontig) return hipErrorInvalidValue;
    const bool full = pair_full_shape<BM, BN>() && gemm_full(d1, BM, BN, BK) && gemm_full(d2, BM, BN, BK);
    const dim3 grid((unsigned)(w1 + w2));
    if (d1.prec == 0) {
        if (full)
            hipLaunchKernelGGL((gemm_pair_kernel<BM, BN, BK, LB, false, false, true, false, true>), grid,
                               dim3(GEMM_THREADS), 0, stream, a1, a2, (int)w1, (int)(w1 + w2));
        else
            hipLaunchKernelGGL((gemm_pair_kernel<BM, BN, BK, LB, false, false, true, false, false>), grid,
                               dim3(GEMM_THREADS), 0, stream, a1, a2, (int)w1, (int)(w1 + w2));
    } else {
        if (full)
            hipLaunchKernelGGL((gemm_pair_bf16_kernel<BM, BN, BK, LB, false, false, true, false, true>), grid,
                               dim3(GEMM_THREADS), 0, stream, a1, a2, (int)w1, (int)(w1 + w2));
        else
            hipLaunchKernelGGL((gemm_pair_bf16_kernel<BM, BN, BK, LB, false, false, true, false, false>), grid,
                               dim3(GEMM_THREADS), 0, stream, a1, a2, (int)w1, (int)(w1 + w2));
    }
    return hipGetLastError();
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// Checks a descriptor and fills the kernel arguments (all but the tile grid).
hipError_t make_args(const GemmDesc &d, GemmArgs &a) {
    if (d.M <= 0 || d.N <= 0 || d.K < 0 || !d.A || !d.B || !d.C) return hipErrorInvalidValue;
    if (d.ksplit < 1 || d.nbo < 1 || d.nbi < 1) return hipErrorInvalidValue;
    if (d.prec < 0 || d.prec > 1 || (d.prec == 1 && (d.causal != CAUSAL_NONE || d.part))) return hipErrorInvalidValue;
    if (d.ksplit > 1 && d.epi != EPI_STORE) return hipErrorInvalidValue;
    // 16-byte vector loads: contiguous extents, leading dims and strides in multiples of 4
    // a K-contiguous operand is read 4 k at a time; an MN-contiguous one row by row
    if (((d.a_kcontig && !d.a_kpad) || d.b_kcontig) && (d.K % 4)) return hipErrorInvalidValue;
    if (d.a_kpad && (!d.a_kcontig || d.lda < (d.K + 3) / 4 * 4)) return hipErrorInvalidValue;
    if ((d.lda % 4) || (d.ldb % 4)) return hipErrorInvalidValue;
    if (!d.a_kcontig && (d.M % 4)) return hipErrorInvalidValue;
    if (!d.b_kcontig && (d.N % 4)) return hipErrorInvalidValue;
    if ((d.sAo % 4) || (d.sAi % 4) || (d.sBo % 4) || (d.sBi % 4)) return hipErrorInvalidValue;
    if (!aligned16(d.A) || !aligned16(d.B)) return hipErrorInvalidValue;
    if ((d.epi == EPI_RESID || d.epi == EPI_GELU_BWD) && !d.aux) return hipErrorInvalidValue;
    if (d.epi == EPI_GELU && !d.C2) return hipErrorInvalidValue;
    if (d.colsum && (d.a_kcontig || d.nbo * d.nbi != 1)) return hipErrorInvalidValue;
    if (d.part && (d.causal != CAUSAL_KEND || d.epi != EPI_STORE || d.ksplit != 1 || d.bias || d.colsum ||
                   d.N % 4 || d.ldc % 4 || d.sCo % 4 || d.sCi % 4 || ((uintptr_t)d.C & 15) || ((uintptr_t)d.part & 15)))
        return hipErrorInvalidValue;

    a = GemmArgs{};
    a.A = d.A; a.B = d.B; a.C = d.C; a.C2 = d.C2; a.bias = d.bias; a.aux = d.aux; a.colsum = d.colsum;
    a.lda = d.lda; a.ldb = d.ldb; a.ldc = d.ldc; a.ldaux = d.ldaux;
    a.sAo = d.sAo; a.sAi = d.sAi; a.sBo = d.sBo; a.sBi = d.sBi; a.sCo = d.sCo; a.sCi = d.sCi;
    a.sCs = d.sCs;
    a.alpha = d.alpha;
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.epi = d.epi; a.causal = d.causal;
    a.nbi = d.nbi; a.ksplit = d.ksplit;
    return hipSuccess;
}

// The tile shape a descriptor runs with (its own, or one picked by size).
int resolve_tile(const GemmDesc &d) {
    if (d.tile != 0) return d.tile;
    const long long batches = (long long)d.nbo * d.nbi * d.ksplit;
    const long long t128 = (long long)((d.M + 127) / 128) * ((d.N + 127) / 128) * batches;
    const long long t64n = (long long)((d.M + 127) / 128) * ((d.N + 63) / 64) * batches;
    if (d.N <= 64) return 2;
    if (t128 >= 512) return 1;
    if (t64n >= 512) return 2;
    return 3;
}

}  // namespace

// The elements a launch for descriptor d may touch, from the operand
// layouts: A(m, k) and B(k, n) over m < M, k < K, n < N in every batch
// (zo < nbo, zi < nbi at strides s?o, s?i), C(m, n) in every batch and split
// (s < ksplit at stride sCs), and the epilogue operands.
static void audit_gemm(AuditSink *au, const char *kernel, const GemmDesc &d) {
    const long long bo = d.nbo - 1, bi = d.nbi - 1, M = d.M, N = d.N, K = d.K;
    if (K > 0) {
        // a K-contiguous A is read 4 k at a time: up to K rounded up to 4 in each row
        const long long ka = d.a_kpad ? (K + 3) / 4 * 4 : K;
        const long long a = (d.a_kcontig ? (M - 1) * d.lda + ka : (K - 1) * d.lda + M) + bo * d.sAo + bi * d.sAi;
        const long long b = (d.b_kcontig ? (N - 1) * d.ldb + K : (K - 1) * d.ldb + N) + bo * d.sBo + bi * d.sBi;
        audit(au, kernel, "A", d.A, a, false);
        audit(au, kernel, "B", d.B, b, false);
    }
    const long long c = (M - 1) * d.ldc + N + bo * d.sCo + bi * d.sCi + (long long)(d.ksplit - 1) * d.sCs;
    audit(au, kernel, "C", d.C, c, true);
    if (d.epi == EPI_GELU) audit(au, kernel, "C2", d.C2, c, true);
    if (d.epi == EPI_RESID || d.epi == EPI_GELU_BWD) audit(au, kernel, "aux", d.aux, (M - 1) * d.ldaux + N, false);
    audit(au, kernel, "bias", d.bias, N, false);
    audit(au, kernel, "colsum", d.colsum, (long long)d.ksplit * M, true);
    if (d.part && d.causal == CAUSAL_KEND) {
        // partial sums of the upper row tiles, [nbo * nbi][M][N], added into C by a second kernel
        audit(au, kernel, "part", d.part, (long long)d.nbo * d.nbi * M * N, true);
        audit(au, "fold_split_sum_kernel", "part", d.part, (long long)d.nbo * d.nbi * M * N, false);
        audit(au, "fold_split_sum_kernel", "C", d.C, c, true);
    }
}

hipError_t gemm_launch(const GemmDesc &d, hipStream_t stream) {
    GemmArgs a;
    hipError_t e = make_args(d, a);
    if (e != hipSuccess) return e;
    if (AuditSink *au = audit_sink()) {
        audit_gemm(au, gemm_kernel_name(d), d);
        return hipSuccess;
    }
    switch (resolve_tile(d)) {
        case 1: return launch_tile<128, 128, 32, 3>(d, a, stream);
        case 2: return launch_tile<128, 64, 32, 3>(d, a, stream);
        case 3: return launch_tile<64, 64, 32, 3>(d, a, stream);
        case 4: return launch_tile<64, 192, 32, 3>(d, a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t gemm_launch_pair(const GemmDesc &d1, const GemmDesc &d2, hipStream_t stream) {
    GemmArgs a1, a2;
    hipError_t e = make_args(d1, a1);
    if (e == hipSuccess) e = make_args(d2, a2);
    if (e != hipSuccess) return e;
    if (d1.tile != d2.tile || d1.causal || d2.causal || d1.prec != d2.prec) return hipErrorInvalidValue;
    if (AuditSink *au = audit_sink()) {
        const char *k = gemm_pair_kernel_name(d1.tile, gemm_pair_full(d1, d2, d1.tile), d1.prec);
        audit_gemm(au, k, d1);
        audit_gemm(au, k, d2);
        return hipSuccess;
    }
    switch (d1.tile) {
        case 1: return launch_pair<128, 128, 32, 3>(d1, a1, d2, a2, stream);
        case 2: return launch_pair<128, 64, 32, 3>(d1, a1, d2, a2, stream);
        case 3: return launch_pair<64, 64, 32, 3>(d1, a1, d2, a2, stream);
    }
    return hipErrorInvalidValue;
}

// Keep in step with the instantiations chosen in gemm_launch and gemm_launch_pair.
const char *gemm_pair_kernel_name(int tile, bool full, int prec) {
    static const char *bf16_names[3][2] = {
        {"gemm_pair_bf16_kernel<128, 128, 32, 3, false, false, true, false, false>",
         "gemm_pair_bf16_kernel<128, 128, 32, 3, false, false, true, false, true>"},
        {"gemm_pair_bf16_kernel<128, 64, 32, 3, false, false, true, false, false>",
         "gemm_pair_bf16_kernel<128, 64, 32, 3, false, false, true, false, true>"},
        {"gemm_pair_bf16_kernel<64, 64, 32, 3, false, false, true, false, false>",
         "gemm_pair_bf16_kernel<64, 64, 32, 3, false, false, true, false, true>"}};
    if (prec) return bf16_names[tile >= 1 && tile <= 3 ? tile - 1 : 0][full ? 1 : 0];
    static const char *names[3][2] = {
        {"gemm_pair_kernel<128, 128, 32, 3, false, false, true, false, false>",
         "gemm_pair_kernel<128, 128, 32, 3, false, false, true, false, true>"},
        {"gemm_pair_kernel<128, 64, 32, 3, false, false, true, false, false>",
         "gemm_pair_kernel<128, 64, 32, 3, false, false, true, false, true>"},
        {"gemm_pair_kernel<64, 64, 32, 3, false, false, true, false, false>",
         "gemm_pair_kernel<64, 64, 32, 3, false, false, true, false, true>"}};
    return names[tile >= 1 && tile <= 3 ? tile - 1 : 0][full ? 1 : 0];
}

bool gemm_pair_full(const GemmDesc &dw, const GemmDesc &di, int tile) {
    static const int bm[3] = {128, 128, 64}, bn[3] = {128, 64, 64};
    const int t = tile >= 1 && tile <= 3 ? tile - 1 : 0;
    return (t == 0 ? pair_full_shape<128, 128>() : t == 1 ? pair_full_shape<128, 64>() : pair_full_shape<64, 64>()) &&
           gemm_full(dw, bm[t], bn[t], 32) && gemm_full(di, bm[t], bn[t], 32);
}

const char *gemm_kernel_name(const GemmDesc &d) {
    static const char *names[4][3][2] = {
        {{"gemm_kernel<128, 128, true, true, 32, 3, false>", "gemm_kernel<128, 128, true, true, 32, 3, true>"},
         {"gemm_kernel<128, 128, true, false, 32, 3, false>", "gemm_kernel<128, 128, true, false, 32, 3, true>"},
         {"gemm_kernel<128, 128, false, false, 32, 3, false>", "gemm_kernel<128, 128, false, false, 32, 3, true>"}},
        {{"gemm_kernel<128, 64, true, true, 32, 3, false>", "gemm_kernel<128, 64, true, true, 32, 3, true>"},
         {"gemm_kernel<128, 64, true, false, 32, 3, false>", "gemm_kernel<128, 64, true, false, 32, 3, true>"},
         {"gemm_kernel<128, 64, false, false, 32, 3, false>", "gemm_kernel<128, 64, false, false, 32, 3, true>"}},
        {{"gemm_kernel<64, 64, true, true, 32, 3, false>", "gemm_kernel<64, 64, true, true, 32, 3, true>"},
         {"gemm_kernel<64, 64, true, false, 32, 3, false>", "gemm_kernel<64, 64, true, false, 32, 3, true>"},
         {"gemm_kernel<64, 64, false, false, 32, 3, false>", "gemm_kernel<64, 64, false, false, 32, 3, true>"}},
        {{"gemm_kernel<64, 192, true, true, 32, 3, false>", "gemm_kernel<64, 192, true, true, 32, 3, true>"},
         {"gemm_kernel<64, 192, true, false, 32, 3, false>", "gemm_kernel<64, 192, true, false, 32, 3, true>"},
         {"gemm_kernel<64, 192, false, false, 32, 3, false>", "gemm_kernel<64, 192, false, false, 32, 3, true>"}}};
    static const char *fold_names[4][3] = {
        {"", "gemm_fold_kernel<128, 128, true, false, 32, 3>", "gemm_fold_kernel<128, 128, false, false, 32, 3>"},
        {"", "gemm_fold_kernel<128, 64, true, false, 32, 3>", "gemm_fold_kernel<128, 64, false, false, 32, 3>"},
        {"", "gemm_fold_kernel<64, 64, true, false, 32, 3>", "gemm_fold_kernel<64, 64, false, false, 32, 3>"},
        {"", "gemm_fold_kernel<64, 192, true, false, 32, 3>", "gemm_fold_kernel<64, 192, false, false, 32, 3>"}};
    static const int bm[4] = {128, 128, 64, 64}, bn[4] = {128, 64, 64, 192};
    const int tile = resolve_tile(d);
    const int t = tile >= 1 && tile <= 4 ? tile - 1 : 0;
    const int l = d.a_kcontig ? (d.b_kcontig ? 0 : 1) : 2;
    static const char *split_names[4][2] = {
        {"gemm_fold_split_kernel<128, 128, true, false, 32, 3, false>",
         "gemm_fold_split_kernel<128, 128, true, false, 32, 3, true>"},
        {"gemm_fold_split_kernel<128, 64, true, false, 32, 3, false>",
         "gemm_fold_split_kernel<128, 64, true, false, 32, 3, true>"},
        {"gemm_fold_split_kernel<64, 64, true, false, 32, 3, false>",
         "gemm_fold_split_kernel<64, 64, true, false, 32, 3, true>"},
        {"gemm_fold_split_kernel<64, 192, true, false, 32, 3, false>",
         "gemm_fold_split_kernel<64, 192, true, false, 32, 3, true>"}};
    static const char *bf16_names[4][3][2] = {
        {{"gemm_bf16_kernel<128, 128, true, true, 32, 3, false>", "gemm_bf16_kernel<128, 128, true, true, 32, 3, true>"},
         {"gemm_bf16_kernel<128, 128, true, false, 32, 3, false>", "gemm_bf16_kernel<128, 128, true, false, 32, 3, true>"},
         {"gemm_bf16_kernel<128, 128, false, false, 32, 3, false>",
          "gemm_bf16_kernel<128, 128, false, false, 32, 3, true>"}},
        {{"gemm_bf16_kernel<128, 64, true, true, 32, 3, false>", "gemm_bf16_kernel<128, 64, true, true, 32, 3, true>"},
         {"gemm_bf16_kernel<128, 64, true, false, 32, 3, false>", "gemm_bf16_kernel<128, 64, true, false, 32, 3, true>"},
         {"gemm_bf16_kernel<128, 64, false, false, 32, 3, false>", "gemm_bf16_kernel<128, 64, false, false, 32, 3, true>"}},
        {{"gemm_bf16_kernel<64, 64, true, true, 32, 3, false>", "gemm_bf16_kernel<64, 64, true, true, 32, 3, true>"},
         {"gemm_bf16_kernel<64, 64, true, false, 32, 3, false>", "gemm_bf16_kernel<64, 64, true, false, 32, 3, true>"},
         {"gemm_bf16_kernel<64, 64, false, false, 32, 3, false>", "gemm_bf16_kernel<64, 64, false, false, 32, 3, true>"}},
        {{"gemm_bf16_kernel<64, 192, true, true, 32, 3, false>", "gemm_bf16_kernel<64, 192, true, true, 32, 3, true>"},
         {"gemm_bf16_kernel<64, 192, true, false, 32, 3, false>", "gemm_bf16_kernel<64, 192, true, false, 32, 3, true>"},
         {"gemm_bf16_kernel<64, 192, false, false, 32, 3, false>",
          "gemm_bf16_kernel<64, 192, false, false, 32, 3, true>"}}};
    if (d.prec) return bf16_names[t][l][gemm_full(d, bm[t], bn[t], 32) ? 1 : 0];
    // causal products with a growing or shrinking K range run with folded row tiles
    if (d.part && d.causal == CAUSAL_KEND && d.M > bm[t] && l == 1)
        return split_names[t][fold_split_full(d, bm[t], bn[t], 32) ? 1 : 0];
    if ((d.causal == CAUSAL_KEND || d.causal == CAUSAL_KSTART) && d.M > bm[t] && l > 0) return fold_names[t][l];
    return names[t][l][gemm_full(d, bm[t], bn[t], 32) ? 1 : 0];
}
