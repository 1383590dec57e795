// Host-side launchers of the 16-bit activation path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// 32-element blocks of x (token-major, nblocks in all) to int16 codes with an
// fp32 scale and an int32 code sum per block.
hipError_t launch_quant_s16(const float* x, int16_t* xq, float* dx, int32_t* sx, int64_t nblocks, hipStream_t s);

// Single-token Q4_K / Q5_K GEMV on 16-bit activation codes; K a multiple of
// 2048 up to 8192. dots != nullptr selects the integer-dot epilogue (int32
// [n, K/32]).
bool s16_gemv_ok(int fmt, int64_t n, int64_t k);
hipError_t launch_kquant_s16(int fmt, const uint8_t* w, const int16_t* xq, const float* dx, const int32_t* sx,
                             float* y, int32_t* dots, int64_t n, int64_t k, hipStream_t s);

}  // namespace qg
