#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// int8-MFMA GEMM for 17..32 tokens (Q4_K and Q6_K weights).
bool mfma_supported(int fmt);
hipError_t launch_gemm32(int fmt, const uint8_t* w, const int8_t* xq, const float* dx, const int32_t* sx,
                         float* y, int64_t n, int64_t k, int m, hipStream_t s);
hipError_t launch_gemm32_dots(int fmt, const uint8_t* w, const int8_t* xq, int32_t* dots, int64_t n,
                              int64_t k, int m, hipStream_t s);

}  // namespace qg
