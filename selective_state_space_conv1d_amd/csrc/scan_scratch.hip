// The static workspace of the allocation-free scan entry point (ssd_chunk_scan_noalloc): the fp16 scan's
// pre-pass tiles for callers that cannot allocate device memory.
#include <mutex>

#include "ssd_kernels.h"

namespace ssd {

// The allocation-free entry point's workspace: a static array, one copy per device (each device's copy
// at its own address), held until the process ends.  Host code never passes the array's name to a
// kernel: it looks the device address up once per device and passes that.
namespace noalloc {
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
}  // namespace noalloc

hipError_t f16_scan_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc::scratch));   // the current device's copy
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = noalloc::kScratchBytes;
    return hipSuccess;
}

}  // namespace ssd
