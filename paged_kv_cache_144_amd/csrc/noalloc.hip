// The fixed device workspace of pa_decode_noalloc (abi.cpp), for callers that cannot
// allocate device memory (code under stream capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The array lives in this file.  In host code its name is only a stand-in for the symbol, so
// noalloc_scratch looks up the array's device address with hipGetSymbolAddress on its first
// call on each device (with that device current) and keeps it per device.  Every call on
// one device shares that device's array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

}  // namespace

namespace pa {

// The array's device address on the current device, looked up once per device.
pa_status noalloc_scratch(void** out, size_t* bytes) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return PA_ERR_LAUNCH;
        }
        addr[dev] = p;
    }
    *out = addr[dev];
    *bytes = kScratchBytes;
    return PA_OK;
}

}  // namespace pa
