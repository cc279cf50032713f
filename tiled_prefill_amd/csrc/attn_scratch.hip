// attn_scratch.hip -- the static device scratch of attn_fwd_noalloc, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array lives in the library's code object: every device the library runs
// on holds its own copy from the module load until the process ends, and no
// call allocates. In host code the array's name is only a stand-in for the
// device symbol, never a device address; the address of this device's copy is
// read once per device with hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_kernels.h"

namespace tpa {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with this device current
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace tpa
