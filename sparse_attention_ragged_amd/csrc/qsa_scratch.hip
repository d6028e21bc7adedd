// Library-owned device scratch for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the split-K
// partials of qsa_sparse_attention_no_alloc live in a file-scope device array instead
// of a caller workspace.
//
// Every GPU the library runs on holds its own copy of the array from the moment the
// code object is loaded on it until the process ends. In host code the array's name
// is only a host-side stand-in, so its device address is looked up once per device
// (with that device current) and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "qsa_host.hpp"

namespace qsa {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

int scratch_address(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev < 0 || dev >= kMaxDevices)
        return (int)hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            // the device whose copy is looked up is the current one (`dev`)
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return (int)e;
            if (!p)
                return (int)hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return 0;
}

}  // namespace qsa
