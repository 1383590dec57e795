#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

// int8-MFMA GEMM for 9..32 tokens over Q4_K and Q6_K weights (K a multiple
// of 256). Activations are already quantized: xqt is the token-tiled copy of
// the codes ([k/32][32][32], gemm32_tiled_act_bytes), dx and block sums sx
// [m, k/32]. When K is split across workgroups (gemm32_partials_bytes > 0)
// the split sums go to `partials` and a second kernel adds them in order
// into y [m, n].
bool mfma_supported(int fmt);
size_t gemm32_partials_bytes(int64_t n, int64_t k);
size_t gemm32_tiled_act_bytes(int64_t k);
hipError_t launch_gemm32(int fmt, const uint8_t* w, const int8_t* xqt, const float* dx, const int32_t* sx,
                         float* y, float* partials, int64_t n, int64_t k, int m, hipStream_t s);
// Checking export: the MFMA integer block dots (Q4_K [m, n, k/32], Q6_K
// [m, n, k/16]) from the token-tiled codes.
hipError_t launch_gemm32_dots(int fmt, const uint8_t* w, const int8_t* xqt, int32_t* dots, int64_t n,
                              int64_t k, int m, hipStream_t s);

}  // namespace qg
