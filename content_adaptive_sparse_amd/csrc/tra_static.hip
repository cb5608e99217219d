// Static device scratch for the entry point that allocates nothing
// (tra_probe_static): callers under HIP graph capture, in tight serving loops
// or in harnesses that forbid hipMalloc.
//
// The array below is a device symbol of this code object.  Its name is only a
// host-side stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and is
// the only form in which host code passes the array anywhere.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tra_internal.h"

namespace tra {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace tra
