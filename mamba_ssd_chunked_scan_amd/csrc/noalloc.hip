// The built-in scratch of ssd_scan_fwd_noalloc: a fixed device array that
// stands in for the caller's workspace, for callers that cannot allocate
// device memory (HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  Each device the library is loaded on holds its own
// copy until the process ends.
#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.hpp"
#include "ssd.h"

namespace ssd {

static __device__ __align__(256) char scratch[SSD_NOALLOC_SCRATCH_BYTES];

// The current device's address of `scratch`, looked up once per device with
// that device current.  In host code the array's name is only a host-side
// stand-in, so this address is what kernels and copies must be given.
hipError_t scratch_ptr(void **out) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace ssd
