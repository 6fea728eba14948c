// Device scratch for the allocation-free drafting entry point
// (dspark_draft_block_noalloc): a fixed array in the library's own device
// memory stands in for the caller's workspace, for callers that cannot
// allocate (code under stream capture, serving loops that forbid it).
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  In host code `scratch` only names the symbol; its device
// address is looked up once per device with that device current and kept
// here, and only that address is ever handed to kernels.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace dspark {

static __device__ __align__(256) uint8_t scratch[kDraftScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t draft_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace dspark
