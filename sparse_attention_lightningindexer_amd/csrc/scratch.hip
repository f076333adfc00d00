// scratch.hip -- per-device state of the library: its own device workspace
// for callers that cannot allocate (HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc), one file-scope device array per GPU of a
// fixed maximum size; and each device's compute-unit count, asked once.
//
// In host code the array's name stands for a host-side shadow, not a device
// address, so the array is only ever reached through the device pointer that
// hipGetSymbolAddress returns.  That lookup is made once per device, with the
// device current, the first time the device asks for its scratch, and the
// pointer is kept per device.  Every call on a GPU shares that GPU's array and
// finds there what the last call left: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.hpp"

namespace dsa {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_for_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t compute_units(int* cus) {
    static std::atomic<int> g_cus[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (n <= 0) return hipErrorInvalidDevice;
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    *cus = n;
    return hipSuccess;
}

}  // namespace dsa
