// Device helpers of the 16-bit activation codes, shared by the 16-bit GEMVs
// and the MoE expert stage.
//
// A 32-element activation block keeps its shape (one fp32 scale) with
// scale = absmax / 32767 and int16 codes rounded half away from zero from
// the IEEE quotient x / scale (the 16-bit activations of "01 · Phase
// overview: from 2B to 8B to MoE", icman.com.cn, issue ledger item ⑫).
#pragma once

#include "common.cuh"

namespace qg {

typedef short s16x2_t __attribute__((ext_vector_type(2)));

// Signed 2 x int16 dot product accumulated into c (v_dot2_i32_i16).
QG_DEV int dot2(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot2(__builtin_bit_cast(s16x2_t, a), __builtin_bit_cast(s16x2_t, b), c, false);
}

// Code of one element for a block scale d > 0.
QG_DEV int code16(float x, float d) {
  const float q = fminf(fmaxf(roundf(x / d), -32767.0f), 32767.0f);
  return (int)q;
}

// A 32-element block of int16 codes in the pairing of the 4-bit code dwords:
// code dword i (bytes 4i .. 4i + 3) holds elements 4i .. 4i + 3 in its low
// nibbles and 16 + 4i .. 16 + 4i + 3 in its high nibbles, and masking it
// with 0x000F000F after shifts of 0, 8, 4 and 12 gives the element pairs
// (4i, 4i + 2), (4i + 1, 4i + 3), (16 + 4i, 16 + 4i + 2),
// (16 + 4i + 1, 16 + 4i + 3); p[4i .. 4i + 3] hold the codes of the same
// pairs. w: the block's codes as 16 dwords of element pairs (2k, 2k + 1).
QG_DEV void pair16(const uint32_t (&w)[16], uint32_t (&p)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[4 * i + 0] = perm(w[2 * i + 1], w[2 * i], 0x05040100u);
    p[4 * i + 1] = perm(w[2 * i + 1], w[2 * i], 0x07060302u);
    p[4 * i + 2] = perm(w[9 + 2 * i], w[8 + 2 * i], 0x05040100u);
    p[4 * i + 3] = perm(w[9 + 2 * i], w[8 + 2 * i], 0x07060302u);
  }
}

// sum over the block of code16 * q for 4-bit codes q (four code dwords).
QG_DEV int q4_dot16(const uint32_t (&q)[4], const uint32_t (&p)[16]) {
  int d = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d = dot2(q[i] & 0x000F000Fu, p[4 * i + 0], d);
    d = dot2((q[i] >> 8) & 0x000F000Fu, p[4 * i + 1], d);
    d = dot2((q[i] >> 4) & 0x000F000Fu, p[4 * i + 2], d);
    d = dot2((q[i] >> 12) & 0x000F000Fu, p[4 * i + 3], d);
  }
  return d;
}

// A block of 16-bit activation codes ready for q4_dot16: paired codes, the
// block scale and the code sum.
struct Act16 {
  uint32_t p[16];
  float dx;
  int sum;
};

}  // namespace qg
