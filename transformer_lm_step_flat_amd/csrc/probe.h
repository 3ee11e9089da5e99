// Calibration kernels (matrix-core and HBM copy rates of the device).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

// One workgroup of 16 wavefronts per CU, each running `iters` rounds of 32
// independent-chain fp32 MFMAs; *flops (host) receives the work launched.
hipError_t probe_mfma(float *out, int iters, hipStream_t s, double *flops);

// dst[0..n) = src[0..n); n % 4 == 0, both 16-byte aligned.
hipError_t probe_copy(float *dst, const float *src, size_t n, hipStream_t s);
