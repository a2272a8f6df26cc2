// fa_noalloc.hip -- the library's own device scratch for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): fa_fwd_splitkv_noalloc keeps its partial states here
// instead of in a caller-supplied workspace.
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the name `scratch` is only a host-side stand-in for the symbol, never
// a device address; the device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is handed to
// kernels.  Calls that overlap on one GPU share the array and race.

#include <hip/hip_runtime.h>

#include <atomic>

#include "fa_internal.h"

namespace fa {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t scratch_address(void **ptr)
{
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // First call on this device (the current one): look the array up.
        // Two threads racing here get the same address.
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace fa
