// Routing helpers shared by the MoE kernels: an order-preserving 64-bit key
// of (logit, expert) and its wave-wide maximum, for top-k selection by
// repeated maxima with ties going to the lower expert index.
#pragma once

#include "common.cuh"

namespace qg {

// Larger logit first, then the lower expert index.
QG_DEV uint64_t route_key(float v, int e) {
  uint32_t b = __float_as_uint(v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(0x7fffffff - e);
}

// The logit a key was made from.
QG_DEV float route_key_value(uint64_t key) {
  uint32_t b = (uint32_t)(key >> 32);
  b = (b & 0x80000000u) ? (b & 0x7fffffffu) : ~b;
  return __uint_as_float(b);
}

QG_DEV int route_key_expert(uint64_t key) { return 0x7fffffff - (int)(uint32_t)key; }

template <int CTRL>
QG_DEV uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}

QG_DEV uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Largest key of the wave, in every lane (DPP within rows of 16, then the
// four rows).
QG_DEV uint64_t wave_max_key(uint64_t k) {
  uint64_t o;
  o = dpp_u64<0xB1>(k); k = o > k ? o : k;    // quad_perm [1,0,3,2]
  o = dpp_u64<0x4E>(k); k = o > k ? o : k;    // quad_perm [2,3,0,1]
  o = dpp_u64<0x141>(k); k = o > k ? o : k;   // row_half_mirror
  o = dpp_u64<0x140>(k); k = o > k ? o : k;   // row_mirror
  const uint64_t r0 = readlane_u64(k, 0), r1 = readlane_u64(k, 16);
  const uint64_t r2 = readlane_u64(k, 32), r3 = readlane_u64(k, 48);
  const uint64_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

}  // namespace qg
