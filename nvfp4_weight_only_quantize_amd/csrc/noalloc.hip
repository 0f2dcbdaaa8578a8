// noalloc.hip -- the device scratch behind qerl_w4a16_lora_gemm_noalloc: a
// file-scope array in the code object, so the call needs neither a workspace
// argument nor any allocation.  Each device that loads the library holds its
// own copy of the array (QERL_NOALLOC_SCRATCH_BYTES) until the process ends.
//
// The array's name is a host-side stand-in in host code; the device address
// of a device's copy comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is handed to kernels.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/qerl.h"
#include "qerl_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[QERL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace qerl {

hipError_t noalloc_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_lock);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace qerl
