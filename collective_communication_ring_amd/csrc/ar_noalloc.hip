// ar_noalloc.hip -- the device memory of the allocation-free all-reduce
// (ar_allreduce_noalloc): one file-scope device array per GPU that stands in
// for the workspace's hand-off region.
//
// The array is part of the library's code object, so the runtime places one
// copy on every GPU the library is loaded on, and each GPU keeps it until the
// process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: the address of a GPU's copy is looked up once per device
// with hipGetSymbolAddress, with that device current, and only that address
// is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ar_internal.h"

namespace ar {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};  // the current device's copy, once looked up
std::mutex g_scratch_mu;

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = kNoAllocScratchBytes;
    return hipSuccess;
}

}  // namespace ar
