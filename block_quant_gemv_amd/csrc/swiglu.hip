// SwiGLU followed by Q8 re-quantization, fused into one pass.
//
// In the FFN sublayer the gate and up projections are computed as one
// GEMV of the shared input (gate rows first); h = silu(gate) * up is then
// re-quantized to 32-element int8 blocks with an fp32 scale for the down
// projection ("Why expert caching can't save dense models", xhh.club,
// single-stream FFN sublayer; "01 · Phase overview: from 2B to 8B to MoE",
// icman.com.cn, stage three: expert gate/up, SwiGLU, down). Eight lanes
// handle one 32-element block of h exactly as the activation quantizer
// does, so h's codes follow the same rule bit for bit.
#include "common.cuh"
#include "swiglu.h"

namespace qg {

// gu: [rows, 2*inter] (row stride gu_ld floats); h: [rows, inter] fp32
// (row stride inter); hq/hd/hs: Q8 blocks of h (row strides inter,
// inter/32, inter/32). rows = tokens (or token x slot pairs).
__global__ __launch_bounds__(256) void swiglu_q8_kernel(const float* __restrict__ gu, int64_t gu_ld,
                                                        float* __restrict__ h, int8_t* __restrict__ hq,
                                                        float* __restrict__ hd, int32_t* __restrict__ hs,
                                                        int64_t rows, int64_t inter) {
  const int64_t nbr = inter / 32;  // blocks per row
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gt >> 3;
  const int part = (int)(gt & 7);
  if (blk >= rows * nbr) return;
  const int64_t r = blk / nbr, b = blk - r * nbr;
  const int64_t col = b * 32 + part * 4;
  const float4 g = *reinterpret_cast<const float4*>(gu + r * gu_ld + col);
  const float4 u = *reinterpret_cast<const float4*>(gu + r * gu_ld + inter + col);
  float4 v;
  v.x = g.x / (1.0f + expf(-g.x)) * u.x;
  v.y = g.y / (1.0f + expf(-g.y)) * u.y;
  v.z = g.z / (1.0f + expf(-g.z)) * u.z;
  v.w = g.w / (1.0f + expf(-g.w)) * u.w;
  *reinterpret_cast<float4*>(h + r * inter + col) = v;
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = max8(a);
  const float d = (a > 0.0f) ? a / 127.0f : 0.0f;
  int s;
  const uint32_t packed = q8_pack4(v, d, s);
  *reinterpret_cast<uint32_t*>(hq + r * inter + col) = packed;
  s = sum4(s);
  s += other_quad(s);
  if (part == 0) {
    hd[r * nbr + b] = d;
    hs[r * nbr + b] = s;
  }
}

hipError_t launch_swiglu_q8(const float* gu, int64_t gu_ld, float* h, int8_t* hq, float* hd,
                            int32_t* hs, int64_t rows, int64_t inter, hipStream_t s) {
  const int64_t threads = rows * (inter / 32) * 8;
  if (threads <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_q8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, gu,
                     gu_ld, h, hq, hd, hs, rows, inter);
  return hipGetLastError();
}

}  // namespace qg
