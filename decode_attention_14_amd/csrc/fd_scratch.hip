// fd_scratch.hip -- the statically allocated workspace of
// fd_decode_attention_noalloc, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops).
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy from the module's load until the process ends, zero-
// filled at load.  In host code its name is only a host-side stand-in, so it
// is never passed to a kernel or a copy; the device address of this GPU's
// copy comes from hipGetSymbolAddress, looked up once per device (with that
// device current) on the first call there, checked, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fd_internal.h"

namespace fdk {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace fdk
