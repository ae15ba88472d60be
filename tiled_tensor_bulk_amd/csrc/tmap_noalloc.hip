// tmap_noalloc.hip -- the status word of tmap_roundtrip_noalloc, the round
// trip for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The copy kernels' only device memory beyond their inputs and outputs is
// one 4-byte status word, which they set when a bounded readiness wait
// expires.  tmap_roundtrip allocates that word with hipMalloc on a device's
// first launch; this entry point uses the word in `scratch` below instead, a
// file-scope device array that exists, zero-initialised, in every device's
// copy of the code object, so that no call here allocates anything.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is asked of the runtime once per device (hipGetSymbolAddress,
// with that device current) and only that address is used afterwards.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "tmap_internal.h"

// The status word of the no-allocation round trip (bit 0: a readiness wait
// expired).  4 bytes per device, held until the process ends; the kernels'
// need for it does not grow with the input, so no input size is refused for
// its sake.
static __device__ __align__(256) uint32_t scratch[1];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint32_t *g_ptr[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up yet)

}  // namespace

// The device address of `scratch` on the current device, looked up on the
// first call there (the caller has passed the library's gfx950 device gate).
tmap_status tmap::noalloc_scratch(uint32_t **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return tmap::record_failure(TMAP_ERROR_UNSUPPORTED_DEVICE, "no HIP device is available");
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            char msg[160];
            std::snprintf(msg, sizeof msg, "cannot look up the status word's device address: %s",
                          hipGetErrorString(e));
            return tmap::record_failure(TMAP_ERROR_LAUNCH, msg);
        }
        g_ptr[dev] = (uint32_t *)p;
    }
    *out = g_ptr[dev];
    return TMAP_SUCCESS;
}

uint32_t *tmap::noalloc_status(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    return g_ptr[dev];
}
