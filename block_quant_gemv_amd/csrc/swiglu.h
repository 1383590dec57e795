#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// h = silu(gu[:, :inter]) * gu[:, inter:2*inter] in fp32, and its Q8 blocks.
hipError_t launch_swiglu_q8(const float* gu, int64_t gu_ld, float* h, int8_t* hq, float* hd,
                            int32_t* hs, int64_t rows, int64_t inter, hipStream_t s);

}  // namespace qg
