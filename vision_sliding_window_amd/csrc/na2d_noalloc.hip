// na2d_noalloc.hip -- the fixed device array behind na2d_backward_noalloc,
// the backward for callers that cannot allocate (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array of NA2D_NOALLOC_SCRATCH_BYTES. Every
// GPU the library runs on holds its own copy, at its own address, until the
// process ends. In host code the array's name is only a host-side stand-in,
// so the device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept; kernels receive that pointer as their
// workspace argument, exactly as na2d_backward passes a caller's workspace.
#include "na2d.h"
#include "na2d_launch.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace na2d {
namespace {

__device__ __align__(256) unsigned char scratch[NA2D_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

}  // namespace

hipError_t noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace na2d
