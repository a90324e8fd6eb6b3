// Temporary: launchers whose kernels are not written yet report hipErrorNotSupported.
#include "launch.hpp"
namespace rf {
hipError_t launch_moe_route(const uint16_t*, const uint16_t*, int64_t, int64_t, int, int, int32_t*, float*, float*,
                            hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quant_rows(const uint16_t*, int64_t, int64_t, uint8_t*, float*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_fp8_gemm(const uint8_t*, const uint8_t*, const float*, const float*, int64_t, int64_t, int64_t,
                           uint16_t*, hipStream_t) { return hipErrorNotSupported; }
}  // namespace rf
