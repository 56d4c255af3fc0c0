// hc_noalloc.hip -- the static device scratch behind hc_fused_step_noalloc.
//
// The fused boundary's kernels need scratch memory for their per-slice partial
// rows (and, for stream counts other than four, the mixes kept between the
// projection and the split). hc_fused_step takes it as a caller-owned workspace;
// the no-allocation variant takes it from this file-scope device array instead,
// so that callers that cannot allocate device memory can still run the boundary.
//
// Each GPU that loads the library holds its own copy of the array, at its own
// address, until the process ends. Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol): the device address
// is looked up once per device with hipGetSymbolAddress, with that device
// current, and that pointer is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hc.h"
#include "hc_internal.h"

namespace hc {
namespace {

__device__ __align__(256) unsigned char scratch[HC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
    *out = nullptr;
    int dev = 0;
    // the stream's device (the null stream belongs to the current one)
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace hc
