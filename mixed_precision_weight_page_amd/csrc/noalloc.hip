// Static device scratch of pw_moe_forward_noalloc, the forward for callers
// that cannot allocate device memory (code under stream capture, tight
// serving loops, harnesses that forbid hipMalloc). One array per device,
// held until the process ends and shared by every call on that device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pw_internal.h"

namespace pw {
namespace {

constexpr uint64_t kScratchBytes = 64ull << 20;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

uint64_t noalloc_scratch_bytes() { return kScratchBytes; }

// The device address of this device's copy of the array. The first call on
// a device (which must be the current device) looks it up; the host-side
// name of the array is not a device address and is never passed on.
hipError_t noalloc_scratch(int device, void** out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_addr[device] = p;
    }
    *out = g_addr[device];
    return hipSuccess;
}

}  // namespace pw
