// SwiGLU followed by Q8 re-quantization, fused into one pass.
//
// In the FFN sublayer the gate and up projections are computed as one
// GEMV of the shared input (gate rows first); h = silu(gate) * up is then
// re-quantized to 32-element int8 blocks with an fp32 scale for the down
// projection ("Why expert caching can't save dense models", xhh.club,
// single-stream FFN sublayer; "01 · Phase overview: from 2B to 8B to MoE",
// icman.com.cn, stage three: expert gate/up, SwiGLU, down). Each 32-element
// block of h is quantized with the activation quantizer's arithmetic, so
// h's codes follow the same rule bit for bit.
#include "common.cuh"
#include "swiglu.h"

namespace qg {

// gu: [rows, 2*inter] (row stride gu_ld floats); h: [rows, inter] fp32
// (row stride inter); hq/hd/hs: Q8 blocks of h (row strides inter,
// inter/32, inter/32). rows = tokens (or token x slot pairs).
// 32 lanes per block, one element each: the block's absolute maximum and
// code sum are 32-lane reductions (DPP within 16 lanes, then one exchange
// between the two rows), and each lane's chain is one SwiGLU and one code.
__global__ __launch_bounds__(256) void swiglu_q8_kernel(const float* __restrict__ gu, int64_t gu_ld,
                                                        float* __restrict__ h, int8_t* __restrict__ hq,
                                                        float* __restrict__ hd, int32_t* __restrict__ hs,
                                                        int64_t rows, int64_t inter) {
  const int64_t nbr = inter / 32;  // blocks per row
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gt >> 5;
  const int el = (int)(gt & 31);
  if (blk >= rows * nbr) return;  // whole 32-lane groups in or out together
  const int64_t r = blk / nbr, b = blk - r * nbr;
  const int64_t col = b * 32 + el;
  const float g = gu[r * gu_ld + col];
  const float u = gu[r * gu_ld + inter + col];
  const float v = g / (1.0f + expf(-g)) * u;
  h[r * inter + col] = v;
  float a = max8(fabsf(v));
  a = fmaxf(a, dpp<0x140>(a));           // 16 lanes (row_mirror)
  a = fmaxf(a, __shfl_xor(a, 16, 64));  // 32 lanes
  const float d = (a > 0.0f) ? a / 127.0f : 0.0f;
  const int q = d != 0.0f ? q8_code(v, d, __builtin_amdgcn_rcpf(d)) : 0;
  hq[r * inter + col] = (int8_t)q;
  int sm = sum4(q);
  sm += other_quad(sm);
  sm += dpp_i<0x140>(sm);          // 16 lanes
  sm += __shfl_xor(sm, 16, 64);    // 32 lanes
  if (el == 0) {
    hd[r * nbr + b] = d;
    hs[r * nbr + b] = sm;
  }
}

hipError_t launch_swiglu_q8(const float* gu, int64_t gu_ld, float* h, int8_t* hq, float* hd,
                            int32_t* hs, int64_t rows, int64_t inter, hipStream_t s) {
  const int64_t threads = rows * (inter / 32) * 32;
  if (threads <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_q8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, gu,
                     gu_ld, h, hq, hd, hs, rows, inter);
  return hipGetLastError();
}

}  // namespace qg
