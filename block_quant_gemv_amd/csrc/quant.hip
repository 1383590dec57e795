// Activation quantizer: fp32 -> 32-element int8 blocks with one fp32 scale.
//
// The method quantizes activations on the device, in real time, to int8
// blocks with an fp32 scale before the quantized dot products ("Why expert
// caching can't save dense models", xhh.club, in-place compute section and
// its Q&A); the scale is the block's absolute maximum over 127 and codes
// round half away from zero. Eight lanes share one block (16 bytes of fp32
// each, one coalesced 128-bit load), reduce the absolute maximum across the
// eight lanes, divide (IEEE fp32 division, as the rule is stated), round
// with roundf (half away from zero) and write 4 codes per lane as one dword.
#include "common.cuh"
#include "internal.h"

namespace qg {

__global__ __launch_bounds__(256) void quant_q8_kernel(const float* __restrict__ x,
                                                       int8_t* __restrict__ xq,
                                                       float* __restrict__ dx,
                                                       int32_t* __restrict__ sx,
                                                       int64_t nblocks) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gt >> 3;
  const int part = (int)(gt & 7);
  // Whole groups of 8 lanes are either all in range or all out of range, so
  // the DPP reductions below always read active partner lanes.
  if (blk >= nblocks) return;
  const float4 v = reinterpret_cast<const float4*>(x)[blk * 8 + part];
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = max8(a);
  const float d = (a > 0.0f) ? a / 127.0f : 0.0f;
  int s;
  const uint32_t packed = q8_pack4(v, d, s);
  reinterpret_cast<uint32_t*>(xq)[blk * 8 + part] = packed;
  s = sum4(s);
  s += other_quad(s);
  if (part == 0) {
    dx[blk] = d;
    if (sx) sx[blk] = s;
  }
}

hipError_t launch_quant_q8(const float* x, int8_t* xq, float* dx, int32_t* sx,
                           int64_t nblocks, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(quant_q8_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, xq, dx, sx,
                     nblocks);
  return hipGetLastError();
}

}  // namespace qg
