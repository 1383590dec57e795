#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

// int8-MFMA GEMM for 9..32 tokens over Q4_K and Q6_K weights (K a multiple
// of 256), one launch. Activations are already quantized, in the
// block-major layout of TiledAct: codes xqt (gemm32_tiled_act_bytes), scales
// dxt [k/32][32] and dx * block sum cxt [k/32][32] (read for Q4_K only);
// token slots m..31 may hold anything. y [m, n].
bool mfma_supported(int fmt);
size_t gemm32_tiled_act_bytes(int64_t k);
hipError_t launch_gemm32(int fmt, const uint8_t* w, const int8_t* xqt, const float* dxt, const float* cxt,
                         float* y, int64_t n, int64_t k, int m, hipStream_t s);
// Checking export: the MFMA integer block dots (Q4_K [m, n, k/32], Q6_K
// [m, n, k/16]) from the block-major codes.
hipError_t launch_gemm32_dots(int fmt, const uint8_t* w, const int8_t* xqt, int32_t* dots, int64_t n,
                              int64_t k, int m, hipStream_t s);

}  // namespace qg
