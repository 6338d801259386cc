// noalloc.hip - rea_decode_step_noalloc: the decode step of include/rea.h run
// in a fixed scratch array that the library holds on every device, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array: the code object reserves it on each
// device the library is loaded on, until the process ends.  In host code its
// name stands for a host-side shadow, not a device address, so the device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to the kernels, as the workspace
// rea_decode_step takes.  The step needs no part of its workspace to start at
// zero: every word a kernel reads was written earlier in the same call.
#include "rea.h"

#include <atomic>
#include <mutex>
#include <stdio.h>

#include "rea_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[REA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];     // device address of scratch, per device
std::mutex g_lookup;

// The device address of `scratch` on the current device `dev`.
hipError_t scratch_on(int dev, void **ptr) {
    if (dev >= 0 && dev < kMaxDevices) {
        void *p = g_scratch[dev].load(std::memory_order_acquire);
        if (p) {
            *ptr = p;
            return hipSuccess;
        }
    }
    std::lock_guard<std::mutex> lock(g_lookup);
    if (dev >= 0 && dev < kMaxDevices) {
        void *p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p) {
            *ptr = p;
            return hipSuccess;
        }
    }
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) g_scratch[dev].store(p, std::memory_order_release);
    *ptr = p;
    return hipSuccess;
}

}  // namespace

extern "C" rea_status rea_decode_step_noalloc(const rea_problem *p, const rea_params *a,
                                              float *out, int32_t *sel, int32_t *n_sel,
                                              void *stream) {
    rea::api_clear_error();
    size_t need = 0;
    rea_status st = rea::decode_check(p, a, out, sel, n_sel, &need);
    if (st != REA_OK) return st;
    if (need > (size_t)REA_NOALLOC_SCRATCH_BYTES) {
        char msg[200];
        snprintf(msg, sizeof(msg),
                 "the step needs %zu bytes of scratch; the fixed array holds %zu "
                 "(rea_decode_step takes a workspace of any size)",
                 need, (size_t)REA_NOALLOC_SCRATCH_BYTES);
        return rea::api_error(REA_EWORKSPACE, msg);
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return rea::api_error(REA_ENODEVICE, "no HIP device available");
    }
    void *ws = nullptr;
    const hipError_t e = scratch_on(dev, &ws);
    if (e != hipSuccess) {
        char msg[200];
        snprintf(msg, sizeof(msg), "hipGetSymbolAddress of the scratch array on device %d: %s",
                 dev, hipGetErrorString(e));
        (void)hipGetLastError();
        return rea::api_error(REA_ENODEVICE, msg);
    }
    return rea::decode_step_ws(p, a, out, sel, n_sel, ws, (size_t)REA_NOALLOC_SCRATCH_BYTES,
                               stream);
}
