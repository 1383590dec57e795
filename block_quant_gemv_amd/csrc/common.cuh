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

// Four dwords at a 2-byte-aligned LDS address in one read: gfx950 serves
// unaligned LDS reads (the compiler emits a single ds_read_b128). Measured on
// MI355X it is slower than lds_read_unaligned's aligned reads plus byte
// shifts in load-bound kernels, and faster where the vector ALU is the bound
// (the IQ4_NL lm_head 4096 -> 248320: 115 -> 111 us sustained).
typedef uint32_t u32x4a2 __attribute__((ext_vector_type(4), aligned(2)));
QG_DEV void lds_read4_direct(const uint8_t* base, uint32_t off, uint32_t (&out)[4]) {
  const u32x4a2 v = *reinterpret_cast<const u32x4a2*>(base + off);
  out[0] = v.x;
  out[1] = v.y;
  out[2] = v.z;
  out[3] = v.w;
}

QG_DEV uint32_t lds_u16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint16_t*>(base + off);
}

// Lane values moved by a DPP pattern. Every pattern used here (quad
// permutes, row mirrors, row rotations) gives every lane a source lane, so
// the bound_ctrl / old-value choice never applies; setting bound_ctrl with a
// zero old value lets the compiler fold the move into a following add
// (v_add_*_dpp).
template <int CTRL>
QG_DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of `width` lanes, width a power of two <= 16; every
// lane of a group ends with its group's sum. DPP steps: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror -- each adds the partner
// half of the next-larger group, so the order of additions is fixed.
QG_DEV float group_sum16(float v, int width) {
  if (width >= 2) v += dpp<0xB1>(v);
  if (width >= 4) v += dpp<0x4E>(v);
  if (width >= 8) v += dpp<0x141>(v);
  if (width >= 16) v += dpp<0x140>(v);
  return v;
}

template <int CTRL>
QG_DEV int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}

// Reductions over aligned groups of 8 lanes (one 32-element block, 4
// elements per lane) with DPP only -- no LDS round trips.
QG_DEV float max8(float v) {
  v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  return fmaxf(v, dpp<0x141>(v));  // row_half_mirror: the other quad
}
// Sum over aligned groups of 4 lanes.
QG_DEV int sum4(int v) {
  v += dpp_i<0xB1>(v);
  return v + dpp_i<0x4E>(v);
}
// Value of the mirrored lane in the other half of an 8-lane group.
QG_DEV int other_quad(int v) { return dpp_i<0x141>(v); }

QG_DEV float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over aligned groups of `width` lanes (power of two <= 64), result in
// every lane of the group. Groups of 32 and 64 add their 16-lane rows with
// lane swaps in a fixed order: (r0 + r1) + (r2 + r3).
QG_DEV float group_sum(float v, int width) {
  v = group_sum16(v, width);
  if (width >= 32) {
    // 16-lane rows 2i and 2i + 1 (v_permlane16_swap gives every lane both).
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  if (width == 64) {
    // The two halves (v_permlane32_swap).
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  }
  return v;
}

// Totals of four rows over a whole wave: each lane holds a partial value of
// rows 0..3 in a0..a3; on return the lanes with l % 4 == r hold row r's
// total. Two exchanges halve the values per lane (lane pairs: odd lanes keep
// rows 1 and 3; then lane quads: lanes with bit 1 set keep rows 2 and 3),
// two row rotations add the lanes of a 16-lane row that hold the same row,
// and two half swaps add the four 16-lane rows. The order of the additions
// is fixed.
QG_DEV float rows4_wave_sum(float a0, float a1, float a2, float a3, int lane) {
  const bool odd = lane & 1;
  const float b0 = (odd ? a1 : a0) + dpp<0xB1>(odd ? a0 : a1);  // quad_perm [1,0,3,2]
  const float b1 = (odd ? a3 : a2) + dpp<0xB1>(odd ? a2 : a3);
  const bool hi = lane & 2;
  float c = (hi ? b1 : b0) + dpp<0x4E>(hi ? b0 : b1);  // quad_perm [2,3,0,1]
  c += dpp<0x124>(c);                                  // row_ror:4
  c += dpp<0x128>(c);                                  // row_ror:8
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(c), __float_as_uint(c), false, false);
  c = __uint_as_float(h[0]) + __uint_as_float(h[1]);  // lanes l and l ^ 32
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(c), __float_as_uint(c), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);  // 16-lane rows 2i and 2i + 1
}

// Totals of two rows over a whole wave (partials in a0, a1); on return the
// lanes with l % 2 == r hold row r's total. Same scheme as rows4_wave_sum
// with one exchange step.
QG_DEV float rows2_wave_sum(float a0, float a1, int lane) {
  const bool odd = lane & 1;
  float c = (odd ? a1 : a0) + dpp<0xB1>(odd ? a0 : a1);  // quad_perm [1,0,3,2]
  c += dpp<0x4E>(c);                                    // quad_perm [2,3,0,1]
  c += dpp<0x124>(c);                                   // row_ror:4
  c += dpp<0x128>(c);                                   // row_ror:8
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(c), __float_as_uint(c), false, false);
  c = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(c), __float_as_uint(c), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
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

// Code of one element: round-half-away(fl32(x / d)), for a block scale
// d = fl32(absmax / 127) > 0 (r = v_rcp(d)). |x| <= absmax, so the code lies
// in -127..127 without a clamp.
//
// fl32(x / d) is the correctly rounded quotient; computing it with the IEEE
// division sequence for every element is the costly part of quantization.
// Instead v' = fl32(x * rcp(d)) is used: v_rcp_f32 is within 1 ulp and the
// product adds half an ulp, so |v' - x/d| <= 1.5 * 2^-23 * |x/d| < 2^-15.4
// (|x/d| <= 127.0001), and fl32(x/d) is within 2^-18 of x/d. Rounding to an
// integer only depends on which side of the nearest half-integer the value
// lies, so whenever v' is at least 2^-14 away from every half-integer the
// code of v' is the code of fl32(x/d); and then v' + copysign(0.5, v') is at
// least 2^-14 away from every integer, so its fp32 sum (error <= 2^-17 below
// 128) truncates to that code. Only within 2^-14 of a half-integer (about 1
// element in 8000) is the exact division taken, rounded by roundf (half away
// from zero). Tiny scales whose reciprocal could leave the normal range also
// take the exact path.
QG_DEV int q8_code(float x, float d, float r) {
  const float v = x * r;
  int q = (int)(v + __builtin_copysignf(0.5f, v));  // truncating conversion
  const float f = __builtin_amdgcn_fractf(fabsf(v));
  if (fabsf(f - 0.5f) < 0x1p-14f || d < 0x1p-100f) q = (int)roundf(x / d);
  return q;
}

// Low bytes of four int32 codes packed little-endian into one dword.
QG_DEV uint32_t pack4_bytes(int q0, int q1, int q2, int q3) {
  const uint32_t lo = perm((uint32_t)q1, (uint32_t)q0, 0x0c0c0400u);  // q0.b0, q1.b0, 0, 0
  const uint32_t hi = perm((uint32_t)q3, (uint32_t)q2, 0x04000c0cu);  // 0, 0, q2.b0, q3.b0
  return lo | hi;
}

// Q8 quantization of 4 consecutive elements of a 32-element block whose
// scale is d = amax / 127 (IEEE division; 0 when amax == 0): codes =
// round-half-away(x / d), all zero when d == 0. Returns the 4 codes packed
// little-endian in one dword and their sum.
QG_DEV uint32_t q8_pack4(float4 v, float d, int& sum) {
  uint32_t packed = 0;
  if (d != 0.0f) {
    const float r = __builtin_amdgcn_rcpf(d);
    packed = pack4_bytes(q8_code(v.x, d, r), q8_code(v.y, d, r), q8_code(v.z, d, r), q8_code(v.w, d, r));
  }
  sum = dot4((int)packed, 0x01010101, 0);
  return packed;
}

}  // namespace qg
