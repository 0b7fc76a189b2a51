// lam_noalloc.hip -- lam_forward_noalloc: lam_forward with its workspace in a
// fixed device array of the library instead of caller memory, for callers
// that cannot allocate (code under graph capture, tight serving loops).
//
// The array lives in device memory for the life of the process, one copy per
// GPU the library runs on.  Its device address is looked up once per device
// with hipGetSymbolAddress and kept; host code uses only that address (the
// array's own name is a host-side stand-in, not a device pointer).  Every
// call on a GPU shares that GPU's copy, so calls that overlap on one GPU race;
// the call's first kernel clears the status word, and the derivation kernel
// overwrites every derived block the scan later reads, so nothing else has to
// start at zero.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lam.h"
#include "lam_internal.h"

namespace {

constexpr size_t kScratchBytes = LAM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];

// Device address of this device's copy of `scratch` (the current device),
// looked up on the first call on that device.
hipError_t scratch_ptr(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" lam_status lam_forward_noalloc(int variant, int dtype, int64_t B, int64_t T, int64_t H,
                                          int64_t dk, int64_t dv, const void *q, const void *k,
                                          const void *v, const void *alpha, const void *erase_b,
                                          const void *write_w, const void *beta,
                                          const float *state_in, void *out, float *state_out,
                                          int algo, hipStream_t stream) {
    size_t need = 0;
    lam_status st = lam_forward_workspace_size(variant, dtype, B, T, H, dk, dv, algo, &need);
    if (st != LAM_OK) return st;
    if (need > kScratchBytes) {
        // auto: the recurrent schedule needs no workspace; an explicit
        // chunked request that does not fit is refused
        if (algo != LAM_ALGO_AUTO) return LAM_ERR_SCRATCH_LIMIT;
        algo = LAM_ALGO_RECURRENT;
        need = 0;
    }
    void *ws = nullptr;
    if (need > 0) {
        if (scratch_ptr(&ws) != hipSuccess) return LAM_ERR_HIP;
    }
    return lam_forward(variant, dtype, B, T, H, dk, dv, q, k, v, alpha, erase_b, write_w, beta,
                       state_in, out, state_out, ws, need ? kScratchBytes : 0, algo, stream);
}
