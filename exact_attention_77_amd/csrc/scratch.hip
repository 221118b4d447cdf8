// scratch.hip -- the library's one fixed device buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, allocation-free
// serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol, not a device address, so
// host code never passes it to a kernel or a copy: it asks the runtime for the
// array's address on the current device once (hipGetSymbolAddress, with that
// device current) and hands that pointer to the kernels.  Every call on one
// GPU shares the array and finds the previous call's contents in it; calls
// that overlap on one GPU (other streams, other host threads) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

namespace fa {

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

int scratch_buffer(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return static_cast<int>(e);
            if (!p) return static_cast<int>(hipErrorInvalidSymbol);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return static_cast<int>(hipSuccess);
}

}  // namespace fa
