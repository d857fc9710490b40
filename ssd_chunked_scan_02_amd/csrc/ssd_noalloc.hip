// The fixed device array behind ssd_forward_noalloc: the forward pass's workspace for callers
// that cannot allocate device memory (code under graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array is a file-scope __device__ variable, so each GPU the library runs on holds its own
// copy from the time the code object is loaded until the process ends.  In host code its name
// is only a host-side stand-in: the device address of this device's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address is
// ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr size_t kNoallocScratchBytes = (size_t)96 << 20;  // 96 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

// The device address of the current device's copy of the scratch array, looked up on the first
// call on each device; null (and *hip_rc set) when the runtime cannot give it.
void* noalloc_scratch(int* hip_rc) {
    *hip_rc = 0;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *hip_rc = e != hipSuccess ? (int)e : -1;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *hip_rc = e != hipSuccess ? (int)e : -1;
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace ssd
