// fp32 MFMA GEMM for gfx950 (v_mfma_f32_32x32x2_f32), LDS-staged tiles.
//
//   C(m, n) <- epi( alpha * sum_k A(m, k) B(k, n) )
//
// Operand layouts (both row-major in memory):
//   a_kcontig: A(m, k) = A[m * lda + k]   else A(m, k) = A[k * lda + m]
//   b_kcontig: B(k, n) = B[n * ldb + k]   else B(k, n) = B[k * ldb + n]
// The three forms used by a linear layer out = in W^T + b (W is out x in):
//   forward  out  = in   W^T : a_kcontig, b_kcontig
//   dinp     dinp = dout W   : a_kcontig, !b_kcontig
//   dweight  dW  += dout^T in: !a_kcontig, !b_kcontig
// The contiguous extent of each operand and every leading dimension must be
// a multiple of 4 and every base pointer 16-byte aligned.
#pragma once
#include <hip/hip_runtime.h>

enum GemmEpi {
    EPI_STORE = 0,    // C = v (+ bias[n])
    EPI_ACCUM = 1,    // C += v
    EPI_RESID = 2,    // C = v (+ bias[n]) + aux[m][n]          (residual add)
    EPI_GELU = 3,     // C = v (+ bias[n]); C2 = gelu(C)          (pre- and post-activation)
    EPI_GELU_BWD = 4  // C = v * gelu'(aux[m][n])                 (gradient through GELU)
};

// Causal handling for the attention products over one (batch, head):
enum GemmCausal {
    CAUSAL_NONE = 0,
    CAUSAL_SKIP_UPPER = 1,  // skip output tiles wholly above the diagonal (n0 >= m0 + BM)
    CAUSAL_KEND = 2,        // reduce only k < m0 + BM (A is zero above the diagonal)
    CAUSAL_KSTART = 3       // reduce only k >= m0 (A(m, k) = X[k][m] with X lower triangular)
};

struct GemmDesc {
    bool a_kcontig = true, b_kcontig = true;
    // a K-contiguous A whose rows continue, zero, to the next multiple of 4
    // (lda at least that): K need not be a multiple of 4
    bool a_kpad = false;
    int M = 0, N = 0, K = 0;
    const float *A = nullptr;
    long long lda = 0;
    const float *B = nullptr;
    long long ldb = 0;
    float *C = nullptr;
    long long ldc = 0;
    float alpha = 1.0f;
    int epi = EPI_STORE;
    const float *bias = nullptr;  // [N] or null
    const float *aux = nullptr;   // [M][ldaux] (EPI_RESID, EPI_GELU_BWD)
    long long ldaux = 0;
    float *C2 = nullptr;          // EPI_GELU post-activation output, leading dim ldc
    int causal = CAUSAL_NONE;
    // batches z = zo * nbi + zi, operand offsets zo * s?o + zi * s?i
    int nbo = 1, nbi = 1;
    long long sAo = 0, sAi = 0, sBo = 0, sBi = 0, sCo = 0, sCi = 0;
    // split-K: partial s goes to C + s * sCs (EPI_STORE only)
    int ksplit = 1;
    long long sCs = 0;
    // Column sums of A (sum over k of A(m, k), m < M), for an MN-contiguous A
    // (the bias gradient of a weight-gradient GEMM): added into colsum[m], or
    // with split-K stored to colsum + s * M.  Computed by the workgroups of the
    // first column of tiles from the A slices already in LDS.
    float *colsum = nullptr;
    // CAUSAL_KEND, EPI_STORE, no bias, ksplit 1: run each folded pair of row
    // tiles as two workgroups, the second one's partial sums of the upper row
    // tiles going to part ([nbo*nbi][M][N] floats) and added into C by a
    // second kernel.
    float *part = nullptr;
    int tile = 0;  // 0 = choose; 1 = 128x128, 2 = 128x64, 3 = 64x64, 4 = 64x192 (not paired)
    // 0: fp32 products; 1: operands rounded to bfloat16 (to nearest even) for
    // the matrix unit, accumulation and everything in memory fp32 (not with
    // causal modes)
    int prec = 0;
};

// Validates the descriptor and enqueues the kernel; returns hipErrorInvalidValue
// for a descriptor the kernel cannot take.
hipError_t gemm_launch(const GemmDesc &d, hipStream_t stream);

// Two independent products in one launch (they share the GPU as one grid, so
// the tail of one is filled by the other): d1 a weight gradient (A and B
// MN-contiguous), d2 an input gradient (A K-contiguous, B MN-contiguous),
// both with the same nonzero `tile` and no causal mode.
hipError_t gemm_launch_pair(const GemmDesc &d1, const GemmDesc &d2, hipStream_t stream);

// The names a kernel-trace profiler shows for the kernels the two calls
// above run with descriptor d (static strings).
const char *gemm_kernel_name(const GemmDesc &d);
const char *gemm_pair_kernel_name(int tile, bool full, int prec);
// Whether gemm_launch_pair runs the pair (weight gradient dw, input gradient
// di) with the kernel for whole tiles and whole K slices.
bool gemm_pair_full(const GemmDesc &dw, const GemmDesc &di, int tile);
