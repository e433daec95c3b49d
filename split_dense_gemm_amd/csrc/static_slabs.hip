// Library-owned slab memory for the entry point that allocates nothing
// (splitk_gemm_bt_auto_noalloc): a file-scope device array, one copy per
// GPU, held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "splitk_internal.h"

static __device__ __attribute__((aligned(256))) float scratch[splitk::kStaticSlabFloats];

namespace splitk {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];
}  // namespace

float* static_slabs() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    float* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
    // Two threads may both look it up; they get the same address.
    g_scratch[dev].store(static_cast<float*>(addr), std::memory_order_release);
    return static_cast<float*>(addr);
}

}  // namespace splitk
