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

// tiled (optional): the block-major copy of the codes, scales and scale *
// block-sum products for the batched matrix-core path (at most 32 tokens).
__global__ __launch_bounds__(256) void quant_q8_kernel(const float* __restrict__ x,
                                                       int8_t* __restrict__ xq,
                                                       float* __restrict__ dx,
                                                       int32_t* __restrict__ sx,
                                                       TiledAct tiled, int64_t nblocks) {
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
  if (tiled.codes) {
    const int t = (int)((uint32_t)blk / (uint32_t)tiled.kblocks);  // blk < 2^32 (checked on launch)
    const int64_t b = blk - (int64_t)t * tiled.kblocks;
    *reinterpret_cast<uint32_t*>(tiled.codes + tiled_code_offset(b, t, 4 * part)) = packed;
    if (part == 0) {
      tiled.dx[b * 32 + t] = d;
      tiled.c[b * 32 + t] = d * (float)s;
    }
  }
  if (part == 0) {
    dx[blk] = d;
    if (sx) sx[blk] = s;
  }
}

hipError_t launch_quant_q8(const float* x, int8_t* xq, float* dx, int32_t* sx,
                           int64_t nblocks, hipStream_t s, const TiledAct* tiled) {
  if (nblocks <= 0) return hipSuccess;
  TiledAct t;
  if (tiled) {
    t = *tiled;
    if (!t.codes || !t.dx || !t.c || t.kblocks <= 0 || nblocks % t.kblocks || nblocks / t.kblocks > 32)
      return hipErrorInvalidValue;
  }
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(quant_q8_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, xq, dx, sx, t, nblocks);
  return hipGetLastError();
}

// Copy of already-quantized codes xq [m, k] into the block-major layout of
// the matrix-core path (m <= 32), for the checking export of that path.
__global__ __launch_bounds__(256) void tile_codes_kernel(const int8_t* __restrict__ xq, int8_t* __restrict__ xqt,
                                                         int m, int kblocks) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 8-byte quarter-block each
  if (gt >= (int64_t)m * kblocks * 4) return;
  const int64_t blk = gt >> 2;
  const int t = (int)(blk / kblocks);
  const int64_t b = blk - (int64_t)t * kblocks;
  const int q = (int)(gt & 3);
  *reinterpret_cast<uint2*>(xqt + tiled_code_offset(b, t, 8 * q)) = reinterpret_cast<const uint2*>(xq)[blk * 4 + q];
}

hipError_t launch_tile_codes(const int8_t* xq, int8_t* xqt, int m, int kblocks, hipStream_t s) {
  if (m < 1 || m > 32 || kblocks < 1) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)m * kblocks * 4;
  hipLaunchKernelGGL(tile_codes_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, xq, xqt, m,
                     kblocks);
  return hipGetLastError();
}

}  // namespace qg
