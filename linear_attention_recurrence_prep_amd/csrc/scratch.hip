// Library-held device scratch for the allocation-free layer-core entry point
// (gdn_layer_core_no_alloc): the same workspace the layer core takes from its
// caller, held instead in a file-scope device array that the code object
// reserves on each device where the library runs, until the process ends.
//
// In host code the array's name stands for a host-side shadow, not a device
// address: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gdn_launch.h"

static __device__ __align__(256) unsigned char scratch[gdn::kScratchBytes];

namespace gdn {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_buffer(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            // with device `dev` current: that device's copy of the array
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace gdn
