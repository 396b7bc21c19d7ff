// The built-in scratch of moe_route_expand_noalloc (api.cpp): for callers
// that may not allocate device memory, the route's workspace -- the histogram
// rows of the multi-workgroup route and, for large batches, the row list of
// the destination-order expand -- lives in a file-scope device array of
// MOE_NOALLOC_SCRATCH_BYTES instead of a caller buffer.  Each GPU the library
// runs on holds its own copy of the array until the process ends.
//
// In host code the array's name is only a stand-in for the symbol: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current), and only that address is ever handed to kernels.
#include "moe_glue.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace moe {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

hipError_t noalloc_scratch(void* stream, void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int cur = 0;
            if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
            if (e != hipSuccess) return e;
            if (r != hipSuccess) return r;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace moe
