// Static device scratch for callers that cannot allocate device memory (code under stream
// capture, tight serving loops): the no-allocation linear forward uses this array instead of a
// workspace from the pool. Each device holds its own copy, at its own address, from the moment
// the library's code object is loaded until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "static_scratch.h"

namespace ep {
namespace {

__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];     // device address of `scratch` per device, once resolved

}  // namespace

// The array's name is a host-side stand-in in host code: its device address comes from the
// runtime, once per device, with that device current.
hipError_t static_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace ep
