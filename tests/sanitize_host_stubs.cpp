// Stand-ins for the kernel launches, for the sanitizer build of the host
// code (tests/test_host_sanitizers.py): every launch reports an error, so a
// call that passes validation returns FD_ERR_DEVICE and touches no device.
#include "fd_internal.h"

namespace fdk {

hipError_t launch_partials(int, int, int, const PartialArgs&, hipStream_t) { return hipErrorNotSupported; }

hipError_t launch_partials_mfma(int, int, const PartialArgs&, hipStream_t) { return hipErrorNotSupported; }

hipError_t launch_combine(int, int, int64_t, int, const float*, const float*, const int32_t*, int64_t, void*,
                          float*, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    return hipErrorNotSupported;
}

hipError_t launch_stream_read(const void*, uint64_t, int, int, uint32_t*, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fdk
