// The library's static device scratch: the workspace of the allocation-free
// decode entry point (mla_decode_partial_noalloc), for callers that cannot
// allocate device memory.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, from module load until the process ends.
// In host code the array's name is only a host-side stand-in for it, never a
// device address, so the host side never passes the name itself anywhere: the
// first call on a device looks up that device's copy with
// hipGetSymbolAddress (with the device current) and every later call reuses
// the address kept for that device.
#include "mla_internal.h"

#include <atomic>
#include <mutex>

namespace mla {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;
}  // namespace

hipError_t scratch_for_current_device(void** ptr) {
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) {
                (void)hipGetLastError();   // the failure is reported by the return value, not left behind
                return e != hipSuccess ? e : hipErrorInvalidSymbol;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace mla
