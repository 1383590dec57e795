// Device helpers shared by the library's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QG_DEV __device__ __forceinline__

namespace qg {

constexpr int kWave = 64;

// Native 128-bit vector (kept in registers; HIP's uint4 wrapper struct can
// block scalar replacement of arrays and push them to scratch).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Signed 4 x int8 dot product accumulated into c (v_dot4 on gfx950).
QG_DEV int dot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

// Bytes [s, s+4) of the 64-bit value {hi:lo}, s in 0..3 (v_alignbyte_b32).
QG_DEV uint32_t alignbyte(uint32_t hi, uint32_t lo, uint32_t s) {
  return __builtin_amdgcn_alignbyte(hi, lo, s);
}

// Byte permute of {hi:lo}: selector byte 0..3 picks a byte of lo, 4..7 of hi.
QG_DEV uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

QG_DEV float half_bits(uint32_t bits16) {
  union { uint16_t u; _Float16 h; } c;
  c.u = (uint16_t)bits16;
  return (float)c.h;
}

// N dwords starting at LDS byte address `off` (any 2-byte alignment). Reads
// N+1 aligned dwords and shifts them into place; up to 3 bytes past the end
// of the requested range are read and discarded.
template <int N>
QG_DEV void lds_read_unaligned(const uint8_t* base, uint32_t off, uint32_t (&out)[N]) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(base + (off & ~3u));
  const uint32_t s = off & 3u;
  uint32_t w[N + 1];
#pragma unroll
  for (int i = 0; i <= N; ++i) w[i] = p[i];
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = alignbyte(w[i + 1], w[i], s);
}

QG_DEV uint32_t lds_u16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint16_t*>(base + off);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
QG_DEV float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

QG_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

QG_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Q8 quantization of 4 consecutive elements of a 32-element block whose
// absolute maximum is `amax`: d = amax / 127 (IEEE division), codes =
// round-half-away(x / d) clamped to +-127; all zero when amax == 0.
// Returns the 4 codes packed little-endian in one dword.
QG_DEV uint32_t q8_pack4(float4 v, float d, int& sum) {
  float e[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed = 0;
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int q = 0;
    if (d != 0.0f) {
      float r = roundf(e[i] / d);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      q = (int)r;
    }
    s += q;
    packed |= ((uint32_t)(q & 0xff)) << (8 * i);
  }
  sum = s;
  return packed;
}

}  // namespace qg
