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

// tanh(u) = 1 - 2 / (exp(2u) + 1): saturates to +-1 through exp's overflow
// and underflow; its absolute error (a few 1e-7) is what matters here.
__device__ __forceinline__ float tanh_fast(float u) { return 1.0f - 2.0f / (__expf(2.0f * u) + 1.0f); }

__device__ __forceinline__ float gelu_fwd(float x) {
    float u = GELU_K * (x + GELU_A * x * x * x);
    return 0.5f * x * (1.0f + tanh_fast(u));
}

// d gelu / dx = 0.5 (1 + tanh u) + 0.5 x (1 - tanh^2 u) k (1 + 3 a x^2)
__device__ __forceinline__ float gelu_grad(float x) {
    float u = GELU_K * (x + GELU_A * x * x * x);
    float th = tanh_fast(u);
    return 0.5f * (1.0f + th) + 0.5f * x * (1.0f - th * th) * GELU_K * (1.0f + 3.0f * GELU_A * x * x);
}

// Rows of the softmax probabilities (and of their gradient) are written as
// exact zeros above the diagonal up to the next multiple of this many
// columns, so that causal GEMM tiles of up to this size can read them.
#define CAUSAL_PAD 128
