// Shared device definitions for the gfx950 kernels of libgpt2mi.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#define WAVE 64

// Lane exchanges inside rows of 16 lanes (DPP): 0xB1 swaps neighbours
// (lane ^ 1), 0x4E swaps pairs (lane ^ 2), 0x141 reverses each half-row of 8
// lanes, 0x140 reverses each row of 16.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wavefront, which must all be active; every lane
// gets the same total.  Each step adds a lane's value to that of a partner
// holding the complementary partial sum (neighbour, pair, mirrored quad,
// mirrored half-row), so after four steps every lane of a row of 16 holds
// the row's sum, bit for bit; the four row sums are then read as scalars
// and added in a fixed order.  No LDS round trips; deterministic.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<0xB1>(v);
    v += dpp_move<0x4E>(v);
    v += dpp_move<0x141>(v);
    v += dpp_move<0x140>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_move<0xB1>(v));
    v = fmaxf(v, dpp_move<0x4E>(v));
    v = fmaxf(v, dpp_move<0x141>(v));
    v = fmaxf(v, dpp_move<0x140>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The values of lanes i mod 32 and i mod 32 + 32, in every lane i: one
// v_permlane32_swap exchanges the two halves of the wavefront in the VALU,
// without the LDS round trip of a general lane shuffle.
__device__ __forceinline__ float2 half_pair(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
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
