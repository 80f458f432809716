// Fixed device scratch for gla_fwd_noalloc: the forward's segment states and
// segment gate totals live in a file-scope device array instead of a caller
// workspace, for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of the array (loaded with
// the code object, kept until the process ends).  In host code the array's
// name is only a stand-in, never a device address: its address on the current
// device is taken once per device with hipGetSymbolAddress and that pointer is
// what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gla_launch.hpp"

namespace gla {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// The scratch array's address on the current device (looked up on the first
// call per device, with that device current).  Returns the HIP error of the
// lookup, or hipErrorInvalidDevice for a device index beyond the table.
hipError_t noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gla
