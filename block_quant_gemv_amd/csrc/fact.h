// Host-side launcher of the float-activation batched GEMV.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Formats with a float-activation kernel: Q4_0 (1) and Q8_0 (2).
bool fact_supported(int fmt);

// y[m, n] = x[m, k] . W_hat^T, fp32 activations, 1 <= m <= 32, k a multiple
// of 32; x 16-byte aligned, w 2-byte aligned.
hipError_t launch_fact(int fmt, const uint8_t* w, const float* x, float* y, int m, int64_t n, int64_t k,
                       hipStream_t s);

}  // namespace qg
