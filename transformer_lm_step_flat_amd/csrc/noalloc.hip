// Entry points that allocate nothing, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid it).  Their kernels keep partial results in `scratch`, a
// file-scope device array of fixed size that each GPU holds from the first
// use until the process ends.
//
// Host code never passes the array's name to a kernel or a copy: in host
// code that name is a host-side stand-in, not a device address.  The device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; only that pointer reaches the kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/gpt2_kernels.h"
#include "kernels.h"
#include "status.h"

namespace {

constexpr size_t kScratchFloats = GPT2K_NOALLOC_SCRATCH_FLOATS;
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float *g_scratch_ptr[kMaxDevices] = {};

gpt2_status fail(gpt2_status st, const std::string &msg) {
    set_last_error(msg);
    return st;
}

// The device address of this device's copy of `scratch` (looked up on the
// first call made with this device current).
hipError_t scratch_for_current_device(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = (float *)p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

gpt2_status gpt2k_layernorm_backward_noalloc(float *dinp, float *dw, float *db, const float *dout, const float *inp,
                                             const float *w, const float *mean, const float *rstd, int N, int C,
                                             int accumulate, void *stream) {
    if (N <= 0 || C <= 0 || C % 4 || C > 2048) return fail(GPT2_EINVAL, "LayerNorm shape not supported");
    if (!dw || !db) return fail(GPT2_EINVAL, "dw and db are required");
    const size_t need = (size_t)ln_partials(N) * 2 * C;
    if (need > kScratchFloats)
        return fail(GPT2_EINVAL, "N * C too large for the static scratch (" + std::to_string(need) +
                                     " floats needed, " + std::to_string(kScratchFloats) + " available)");
    float *ws = nullptr;
    hipError_t e = scratch_for_current_device(&ws);
    if (e != hipSuccess) return fail(GPT2_EDEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    // every partial row is written by one workgroup before the sum kernel
    // reads it, so the scratch needs no clearing
    e = k_layernorm_backward(dinp, dw, db, ws, dout, inp, w, mean, rstd, N, C, accumulate != 0, (hipStream_t)stream);
    if (e == hipErrorInvalidValue) return fail(GPT2_EINVAL, "LayerNorm shape not supported");
    if (e != hipSuccess) return fail(GPT2_EDEVICE, std::string("layernorm backward: ") + hipGetErrorString(e));
    return GPT2_OK;
}

}  // extern "C"
