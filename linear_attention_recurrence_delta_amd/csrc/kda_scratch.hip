// kda_scratch.hip -- the library's one static device buffer, for callers that
// cannot allocate (kda_prefill_ex_noalloc in include/kda.h).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in; its device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current and kept here, and that address is the only one handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

__device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device, once taken

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
