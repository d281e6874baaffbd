// Device scratch owned by the library, for himuon_tiled_ns_noalloc: callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc) run the step-by-step path
// through this fixed array instead of a workspace of their own.
//
// The array is a file-scope __device__ object: the HIP runtime places one copy
// on every device the library runs on, when it loads the code object there,
// and keeps it until the process ends.  In host code its name is only a
// host-side stand-in; the device address of each copy comes from
// hipGetSymbolAddress with that device current, taken once per device and
// kept here.  Only those addresses are ever handed to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"

static __device__ __align__(256) unsigned char scratch[himuon::kStaticScratchBytes];

namespace himuon {

hipError_t static_scratch(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace himuon
