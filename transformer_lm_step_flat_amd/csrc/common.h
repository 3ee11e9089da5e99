// Shared device definitions for the gfx950 kernels of libgpt2mi.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#define WAVE 64

// Sum over the 64 lanes of a wavefront; every lane gets the total.  The
// butterfly order is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// tanh-approximate GELU, 0.5 x (1 + tanh(k (x + 0.044715 x^3))), k = sqrt(2/pi).
#define GELU_K 0.7978845608028654f
#define GELU_A 0.044715f

// With r = 1 / (exp(2u) + 1), tanh u = 1 - 2r, so 0.5 (1 + tanh u) = 1 - r and
// 1 - tanh^2 u = 4 r (1 - r).  r saturates to 0 or 1 through exp's overflow
// and underflow; its absolute error (a few 1e-7) is what matters here.
__device__ __forceinline__ float gelu_r(float x, float x2) {
    const float u = GELU_K * x * (1.0f + GELU_A * x2);
    // the hardware reciprocal (about 1 ulp): exp(2u) + 1 >= 1, and 1 / inf = 0
    return __builtin_amdgcn_rcpf(__expf(2.0f * u) + 1.0f);
}

// gelu(x) = x (1 - r)
__device__ __forceinline__ float gelu_fwd(float x) { return x * (1.0f - gelu_r(x, x * x)); }

// d gelu / dx = 0.5 (1 + tanh u) + 0.5 x (1 - tanh^2 u) k (1 + 3 a x^2)
//             = (1 - r) (1 + 2 x r k (1 + 3 a x^2))
__device__ __forceinline__ float gelu_grad(float x) {
    const float x2 = x * x;
    const float r = gelu_r(x, x2);
    return (1.0f - r) * (1.0f + 2.0f * x * r * (GELU_K + 3.0f * GELU_A * GELU_K * x2));
}

// Rows of the softmax probabilities (and of their gradient) are written as
// exact zeros above the diagonal up to the next multiple of this many
// columns, so that causal GEMM tiles of up to this size can read them.
#define CAUSAL_PAD 128
