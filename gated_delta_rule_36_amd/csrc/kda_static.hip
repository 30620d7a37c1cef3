// Fixed device scratch for kda_fwd_scan_static: the segmented form's end
// states and transition matrices, for callers that cannot allocate device
// memory.  One array per GPU (the code object is loaded once per device),
// held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

// The array's name is a host-side stand-in in host code: its device address
// on each GPU comes from hipGetSymbolAddress, with that GPU current.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

hipError_t static_scratch(void **ptr)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
