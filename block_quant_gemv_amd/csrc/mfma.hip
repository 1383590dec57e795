#include "mfma.h"

namespace qg {

bool mfma_supported(int) { return false; }
hipError_t launch_gemm32(int, const uint8_t*, const int8_t*, const float*, const int32_t*, float*, int64_t,
                         int64_t, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_gemm32_dots(int, const uint8_t*, const int8_t*, int32_t*, int64_t, int64_t, int,
                              hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace qg
