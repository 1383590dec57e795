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

// Grouped single-token Q4_0 GEMV on 16-bit codes for the MoE experts: one
// problem per grouping-table entry (see internal.h; one token per entry).
struct S16Grouped {
  const uint8_t* w = nullptr;         // expert matrices, w_stride bytes apart
  int64_t w_stride = 0;
  const uint8_t* w_shared = nullptr;  // shared expert (entry expert == -1)
  const int32_t* tbl = nullptr;
  int tbl_stride = 0;
  int nprob = 0;                      // grid entries (tbl[0] of them in use)
  const int16_t* xq = nullptr;        // codes [rows][xs], scales/sums [rows][xs/32]
  const float* dx = nullptr;
  const int32_t* sx = nullptr;
  int64_t xs = 0;
  int act_div = 1;
  float* y = nullptr;
  int64_t ldy = 0;
  int64_t n = 0, k = 0;
};
bool q40_s16_grouped_ok(int64_t k);  // K = 512, 1024, 2048 or 4096
hipError_t launch_q40_s16_grouped(const S16Grouped& a, hipStream_t s);
// h = silu(gate) * up and its 16-bit blocks (hq int16, hd fp32, hs int32).
hipError_t launch_swiglu_s16(const float* gu, int64_t gu_ld, float* h, int16_t* hq, float* hd, int32_t* hs,
                             int64_t rows, int64_t inter, hipStream_t s);

}  // namespace qg
