// Calibration kernels for the measurement: the fp32 matrix-core rate and the
// HBM copy rate this device reaches, reported beside the vendor peaks.
#include "common.h"
#include "probe.h"

namespace {

constexpr int PROBE_THREADS = 1024;  // 16 wavefronts: 4 per SIMD
constexpr int PROBE_CHAINS = 4;      // independent accumulators per wavefront
constexpr int PROBE_UNROLL = 8;

// Back-to-back v_mfma_f32_32x32x2_f32 on register operands only.  The sum of
// the accumulators is written only if it equals a value it cannot take, so
// the work is kept without a store per thread.
__global__ __launch_bounds__(PROBE_THREADS) void mfma_probe_kernel(float *out, int iters) {
    floatx16 acc[PROBE_CHAINS];
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[c][r] = 0.0f;
    const float a = (float)(threadIdx.x & 63) * 1e-3f, b = 1.0f + (float)(threadIdx.x >> 6) * 1e-4f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < PROBE_UNROLL; k++)
#pragma unroll
            for (int c = 0; c < PROBE_CHAINS; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; c++)
#pragma unroll
        for (int r = 0; r < 16; r++) s += acc[c][r];
    if (s == -1.0f) out[0] = s;  // never true: a, b >= 0
}

// dst = src, float4 per thread, 4 per workgroup round, non-temporal.
__global__ __launch_bounds__(256) void copy_probe_kernel(floatx4 *dst, const floatx4 *src, size_t n4) {
    const size_t base = (size_t)blockIdx.x * 1024 + threadIdx.x;
    floatx4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++)
        if (base + (size_t)u * 256 < n4) v[u] = __builtin_nontemporal_load(src + base + (size_t)u * 256);
#pragma unroll
    for (int u = 0; u < 4; u++)
        if (base + (size_t)u * 256 < n4) __builtin_nontemporal_store(v[u], dst + base + (size_t)u * 256);
}

}  // namespace

hipError_t probe_mfma(float *out, int iters, hipStream_t s, double *flops) {
    if (!out || iters < 1) return hipErrorInvalidValue;
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (ncu < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(ncu), dim3(PROBE_THREADS), 0, s, out, iters);
    if (flops)
        *flops = 2.0 * 32 * 32 * 2 * (double)PROBE_UNROLL * PROBE_CHAINS * iters * (PROBE_THREADS / 64) * ncu;
    return hipGetLastError();
}

hipError_t probe_copy(float *dst, const float *src, size_t n, hipStream_t s) {
    if (!dst || !src || n % 4 || (((uintptr_t)dst | (uintptr_t)src) & 15)) return hipErrorInvalidValue;
    const size_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    if ((n4 + 1023) / 1024 > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)((n4 + 1023) / 1024)), dim3(256), 0, s, (floatx4 *)dst,
                       (const floatx4 *)src, n4);
    return hipGetLastError();
}
