// Device scratch of the entry point that allocates nothing (ra_ring_fwd_noalloc).
//
// A file-scope device array: every GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code the array's name is only a
// host-side stand-in, never a device address: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current (on the first
// call on that device) and kept per device.  Calls on one GPU share that GPU's copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ra_internal.h"

namespace ra {
namespace {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_region(void** ptr, size_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kNoAllocScratchBytes;
    return hipSuccess;
}

}  // namespace ra
