#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

// int8-MFMA GEMM for 17..32 tokens over Q4_K and Q6_K weights (K a multiple
// of 256). Activations are already quantized (xq [m, k], dx and block sums
// sx [m, k/32]). Split-K partial sums go to `partials`
// (gemm32_partials_bytes) and are added in a fixed order into y [m, n].
bool mfma_supported(int fmt);
size_t gemm32_partials_bytes(int64_t n, int64_t k);
hipError_t launch_gemm32(int fmt, const uint8_t* w, const int8_t* xq, const float* dx, const int32_t* sx,
                         float* y, float* partials, int64_t n, int64_t k, int m, hipStream_t s);
// Checking export: the MFMA integer block dots (Q4_K [m, n, k/32], Q6_K
// [m, n, k/16]).
hipError_t launch_gemm32_dots(int fmt, const uint8_t* w, const int8_t* xq, int32_t* dots, int64_t n,
                              int64_t k, int m, hipStream_t s);

}  // namespace qg
