// Host-only stand-ins for the kernel launchers and the one HIP runtime call
// of the C-ABI front end, so that api.cpp's argument validation can be built
// and run under AddressSanitizer / UndefinedBehaviorSanitizer on a machine
// without a GPU.  Every launcher reports an error: a call that got past the
// validation would show up as TE_ERR_HIP, never as a launch.
#include <hip/hip_runtime_api.h>

#include "internal.h"

extern "C" const char* hipGetErrorString(hipError_t) { return "host sanitizer build: no device"; }

namespace tefp8 {
int device_cus() { return 256; }
hipError_t launch_gemm(const GemmArgs&, hipStream_t, LaunchInfo*) { return hipErrorNoDevice; }
hipError_t launch_zero_f32(float*, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bgrad_reduce(const float*, int64_t, int64_t, int64_t, float*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_mgrouped_bgrad_reduce(const float*, int64_t, int64_t, int64_t, int32_t, const int32_t*, float*,
                                        hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t noalloc_scratch(void**) { return hipErrorNoDevice; }
hipError_t launch_cast(const uint16_t*, int64_t, int64_t, int64_t, int, bool, uint8_t*, int64_t, float*, int64_t,
                       hipStream_t, LaunchInfo*) { return hipErrorNoDevice; }
hipError_t launch_row_sum(const uint8_t*, int64_t, int64_t, int64_t, int, const float*, int64_t, float*, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_cast_batch(const CastOperand*, int, int, bool, hipStream_t, LaunchInfo*) { return hipErrorNoDevice; }
hipError_t launch_cast_transpose(const uint16_t*, int64_t, int64_t, int64_t, int, bool, uint8_t*, int64_t, float*,
                                 int64_t, uint8_t*, int64_t, float*, int64_t, hipStream_t, LaunchInfo*)
{
    return hipErrorNoDevice;
}
}  // namespace tefp8
