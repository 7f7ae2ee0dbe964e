// Stand-ins for the kernel launchers and the few HIP runtime calls of the
// library's host code, so capi.cpp, chooser.cpp and bank_model.cpp can be
// built with the address and undefined-behaviour sanitizers and exercised
// on a machine without a GPU (tests/test_sanitized_host.py).  TEST
// INFRASTRUCTURE ONLY: every launcher reports success without doing
// anything, and the event calls report that no device is present.
#include <hip/hip_runtime_api.h>

#include "launch.h"

namespace swz {

hipError_t launch_convert(int, const ConvertJob&, hipStream_t) { return hipSuccess; }
hipError_t launch_rows(int, const ConvertJob&, hipStream_t) { return hipSuccess; }
hipError_t launch_stage(const StageJob&, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm_frag(const void*, const void*, float*, int64_t, int64_t, int64_t, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_gemm_tiles(const void*, const void*, void*, int64_t, int64_t, int64_t, const LdsLayout&, bool,
                             hipStream_t) {
    return hipSuccess;
}
hipError_t launch_map(const int32_t*, int32_t*, int64_t, swz_params, hipStream_t) { return hipSuccess; }
hipError_t launch_map_batch(const int32_t*, int32_t*, int64_t, const MapParamPack&, int, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_copy(const void*, void*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_lds_probe(const uint32_t*, const uint64_t*, int, int, bool, int, int, uint64_t*, hipStream_t) {
    return hipSuccess;
}

}  // namespace swz

hipError_t hipEventCreate(hipEvent_t* e) {
    *e = nullptr;
    return hipErrorNoDevice;
}
hipError_t hipEventDestroy(hipEvent_t) { return hipErrorNoDevice; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipErrorNoDevice; }
hipError_t hipEventElapsedTime(float*, hipEvent_t, hipEvent_t) { return hipErrorNoDevice; }
