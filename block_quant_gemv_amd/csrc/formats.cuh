// Device-side views of the packed block formats and of the staged Q8
// activations, shared by the decode GEMV and the MoE expert kernels.
//
// Each format struct reads one 32-element unit of a block (or one
// 32-element sub-block of a 256-element super-block) from LDS at any 2-byte
// alignment, decodes it to int8 lanes in registers -- codes as they are, the
// K-quant scale and min fields, or the non-linear format's 16-entry codebook
// looked up with byte permutes -- and combines it with a unit of Q8
// activations by 4-way int8 dot products, then scales in fp32 ("Why expert
// caching can't save dense models", xhh.club, Q&A on computing GGUF blocks
// without FP16 expansion).
#pragma once

#include "common.cuh"
#include "internal.h"

namespace qg {

// ------------------------------------------------------------ activations --

struct Act {
  int x[8];     // 32 int8 codes, element order
  float dx;     // block scale
  int sa, sb;   // sums of codes 0..15 and 16..31
};

QG_DEV Act load_act(const uint8_t* tok, int U, int u) {
  Act a;
  const int4 lo = *reinterpret_cast<const int4*>(tok + 16 * u);
  const int4 hi = *reinterpret_cast<const int4*>(tok + 16 * U + 16 * u);
  const int2 mt = *reinterpret_cast<const int2*>(tok + 32 * U + 8 * u);
  a.x[0] = lo.x; a.x[1] = lo.y; a.x[2] = lo.z; a.x[3] = lo.w;
  a.x[4] = hi.x; a.x[5] = hi.y; a.x[6] = hi.z; a.x[7] = hi.w;
  a.dx = __int_as_float(mt.x);
  a.sa = (int)(int16_t)(mt.y & 0xffff);
  a.sb = mt.y >> 16;
  return a;
}

__host__ __device__ constexpr int act_token_bytes(int U) { return (40 * U + 15) / 16 * 16; }

// ---------------------------------------------------------------- formats --

struct FmtQ4_0 {
  static constexpr int kUPB = 1, kBB = 18;
  struct W { uint32_t q[4]; float d; };
  QG_DEV static W load(const uint8_t* t, uint32_t off, int, const uint32_t*) {
    W w;
    w.d = half_bits(lds_u16(t, off));
    lds_read_unaligned<4>(t, off + 2, w.q);
    return w;
  }
  // sum xq * (q - 8)
  QG_DEV static int idot(const W& w, const Act& a) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = dot4((int)(w.q[i] & 0x0F0F0F0Fu), a.x[i], s);
      s = dot4((int)((w.q[i] >> 4) & 0x0F0F0F0Fu), a.x[4 + i], s);
    }
    return s - 8 * (a.sa + a.sb);
  }
  QG_DEV static float fma(const W& w, const Act& a, float acc) {
    return fmaf((float)idot(w, a), a.dx * w.d, acc);
  }
  QG_DEV static void dots(const W& w, const Act& a, int32_t* out) { out[0] = idot(w, a); }
  static constexpr int kDotsPerUnit = 1;
};

struct FmtQ8_0 {
  static constexpr int kUPB = 1, kBB = 34;
  struct W { uint32_t q[8]; float d; };
  QG_DEV static W load(const uint8_t* t, uint32_t off, int, const uint32_t*) {
    W w;
    w.d = half_bits(lds_u16(t, off));
    lds_read_unaligned<8>(t, off + 2, w.q);
    return w;
  }
  QG_DEV static int idot(const W& w, const Act& a) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot4((int)w.q[i], a.x[i], s);
    return s;
  }
  QG_DEV static float fma(const W& w, const Act& a, float acc) {
    return fmaf((float)idot(w, a), a.dx * w.d, acc);
  }
  QG_DEV static void dots(const W& w, const Act& a, int32_t* out) { out[0] = idot(w, a); }
  static constexpr int kDotsPerUnit = 1;
};

// Codebook lookup of the 8 nibble codes of one dword (low nibbles -> vlo,
// high nibbles -> vhi, byte i of each from byte i of q). cb holds two
// 8-byte pools built by the host: L (cb[0], cb[1]) serves codes 0..7 at
// byte-permute selector n, H (cb[2], cb[3]) codes 8..15 at selector n ^ 8,
// and the entry is the xor of the two permutes. For a code of the other
// half a selector lands in 8..15, where the permute yields a fill byte
// (sign of pool byte 1/3/5/7, 0x00, or 0xFF) instead of a pool byte; every
// pool byte is stored xor-ed with the fill its code meets in the other pool.
// Two permutes and an xor per four codes, no bit-3 pick.
QG_DEV void cb_lookup8(uint32_t q, const uint32_t* cb, uint32_t& vlo, uint32_t& vhi) {
  const uint32_t s0 = q & 0x0F0F0F0Fu, s1 = (q >> 4) & 0x0F0F0F0Fu;
  vlo = perm(cb[1], cb[0], s0) ^ perm(cb[3], cb[2], s0 ^ 0x08080808u);
  vhi = perm(cb[1], cb[0], s1) ^ perm(cb[3], cb[2], s1 ^ 0x08080808u);
}

struct FmtIQ4_NL {
  static constexpr int kUPB = 1, kBB = 18;
  struct W { uint32_t v[8]; float d; };
  QG_DEV static W load(const uint8_t* t, uint32_t off, int, const uint32_t* cb) {
    W w;
    uint32_t q[4];
    w.d = half_bits(lds_u16(t, off));
    lds_read4_direct(t, off + 2, q);  // no byte shifts: this decode is ALU-bound
#pragma unroll
    for (int i = 0; i < 4; ++i) cb_lookup8(q[i], cb, w.v[i], w.v[4 + i]);
    return w;
  }
  QG_DEV static int idot(const W& w, const Act& a) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot4((int)w.v[i], a.x[i], s);
    return s;
  }
  QG_DEV static float fma(const W& w, const Act& a, float acc) {
    return fmaf((float)idot(w, a), a.dx * w.d, acc);
  }
  QG_DEV static void dots(const W& w, const Act& a, int32_t* out) { out[0] = idot(w, a); }
  static constexpr int kDotsPerUnit = 1;
};

struct FmtQ4_K {
  static constexpr int kUPB = 8, kBB = 144;
  struct W { uint32_t q[4]; float dsc, dmm; };
  // off = byte offset of the super-block (16-byte aligned), g = sub-block.
  QG_DEV static W load(const uint8_t* t, uint32_t off, int g, const uint32_t*) {
    W w;
    const uint4 h = *reinterpret_cast<const uint4*>(t + off);
    const uint4 q = *reinterpret_cast<const uint4*>(t + off + 16 + 16 * g);
    w.q[0] = q.x; w.q[1] = q.y; w.q[2] = q.z; w.q[3] = q.w;
    const float d = half_bits(h.x & 0xffffu);
    const float dmin = half_bits(h.x >> 16);
    const uint64_t s_lo = (uint64_t)h.y | ((uint64_t)h.z << 32);   // stream bits 0..63
    const uint64_t s_hi = (uint64_t)h.z | ((uint64_t)h.w << 32);   // stream bits 32..95
    const uint32_t sc = (uint32_t)(s_lo >> (6 * g)) & 63u;
    const uint32_t mn = (uint32_t)(s_hi >> (16 + 6 * g)) & 63u;
    w.dsc = d * (float)sc;
    w.dmm = dmin * (float)mn;
    return w;
  }
  // sum xq * q (codes 0..15)
  QG_DEV static int idot(const W& w, const Act& a) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = dot4((int)(w.q[i] & 0x0F0F0F0Fu), a.x[i], s);
      s = dot4((int)((w.q[i] >> 4) & 0x0F0F0F0Fu), a.x[4 + i], s);
    }
    return s;
  }
  QG_DEV static float fma(const W& w, const Act& a, float acc) {
    acc = fmaf(a.dx * w.dsc, (float)idot(w, a), acc);
    return fmaf(-(a.dx * w.dmm), (float)(a.sa + a.sb), acc);
  }
  QG_DEV static void dots(const W& w, const Act& a, int32_t* out) { out[0] = idot(w, a); }
  static constexpr int kDotsPerUnit = 1;
};

// Q4_K with a fifth code bit: sub-block j's fifth bits are the word
// qh[4j..4j+3], element i (0..31) at bit 8 (i % 4) + i / 4. The four codes of
// code dword i (elements 4i..4i+3, low nibbles) then take bit i of each
// byte, and those of the high nibbles (elements 16 + 4i ..) bit 4 + i: one
// shift and one mask move four fifth bits to bit 4 of their bytes.
struct FmtQ5_K {
  static constexpr int kUPB = 8, kBB = 176;
  struct W { uint32_t c[8]; float dsc, dmm; };
  QG_DEV static W load(const uint8_t* t, uint32_t off, int g, const uint32_t*) {
    W w;
    const uint4 h = *reinterpret_cast<const uint4*>(t + off);
    const uint32_t qh = *reinterpret_cast<const uint32_t*>(t + off + 16 + 4 * g);
    const uint4 q = *reinterpret_cast<const uint4*>(t + off + 48 + 16 * g);
    const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w.c[i] = (qq[i] & 0x0F0F0F0Fu) | ((qh << (4 - i)) & 0x10101010u);
      w.c[4 + i] = ((qq[i] >> 4) & 0x0F0F0F0Fu) | ((qh >> i) & 0x10101010u);
    }
    const float d = half_bits(h.x & 0xffffu);
    const float dmin = half_bits(h.x >> 16);
    const uint64_t s_lo = (uint64_t)h.y | ((uint64_t)h.z << 32);
    const uint64_t s_hi = (uint64_t)h.z | ((uint64_t)h.w << 32);
    w.dsc = d * (float)((uint32_t)(s_lo >> (6 * g)) & 63u);
    w.dmm = dmin * (float)((uint32_t)(s_hi >> (16 + 6 * g)) & 63u);
    return w;
  }
  // sum xq * q (codes 0..31)
  QG_DEV static int idot(const W& w, const Act& a) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot4((int)w.c[i], a.x[i], s);
    return s;
  }
  QG_DEV static float fma(const W& w, const Act& a, float acc) {
    acc = fmaf(a.dx * w.dsc, (float)idot(w, a), acc);
    return fmaf(-(a.dx * w.dmm), (float)(a.sa + a.sb), acc);
  }
  QG_DEV static void dots(const W& w, const Act& a, int32_t* out) { out[0] = idot(w, a); }
  static constexpr int kDotsPerUnit = 1;
};

// IQ4_NL codes on a 256-element super-block with 6-bit sub-scales: header
// d | scales_h | scales_l[4] (8 bytes), then sub-block j's 16 code bytes at
// 8 + 16 j. Super-blocks (136 B) are 8-byte aligned in every step.
struct FmtIQ4_XS {
  static constexpr int kUPB = 8, kBB = 136;
  struct W { uint32_t v[8]; float ds; };
  QG_DEV static W load(const uint8_t* t, uint32_t off, int g, const uint32_t* cb) {
    W w;
    const uint2 h = *reinterpret_cast<const uint2*>(t + off);
    const uint2 qa = *reinterpret_cast<const uint2*>(t + off + 8 + 16 * g);
    const uint2 qb = *reinterpret_cast<const uint2*>(t + off + 16 + 16 * g);
    const uint32_t q[4] = {qa.x, qa.y, qb.x, qb.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) cb_lookup8(q[i], cb, w.v[i], w.v[4 + i]);
    const uint32_t ls = ((h.y >> (4 * g)) & 0xFu) | (((h.x >> (16 + 2 * g)) & 3u) << 4);
    w.ds = half_bits(h.x & 0xffffu) * (float)((int)ls - 32);
    return w;
  }
  QG_DEV static int idot(const W& w, const Act& a) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot4((int)w.v[i], a.x[i], s);
    return s;
  }
  QG_DEV static float fma(const W& w, const Act& a, float acc) {
    return fmaf((float)idot(w, a), a.dx * w.ds, acc);
  }
  QG_DEV static void dots(const W& w, const Act& a, int32_t* out) { out[0] = idot(w, a); }
  static constexpr int kDotsPerUnit = 1;
};

struct FmtQ6_K {
  static constexpr int kUPB = 8, kBB = 210;
  struct W { uint32_t c[8]; float d; int sca, scb; };
  // High 2 bits of the 4 codes in code dword w sit at bits 2*(w/2) of the
  // bytes of qh dword (w & 1); move them to bits 4..5.
  QG_DEV static uint32_t hi2(uint32_t qh, int k) {
    const uint32_t v = (k == 0) ? (qh << 4) : (k == 1) ? (qh << 2) : (k == 2) ? qh : (qh >> 2);
    return v & 0x30303030u;
  }
  QG_DEV static W load(const uint8_t* t, uint32_t off, int g, const uint32_t*) {
    W w;
    w.d = half_bits(lds_u16(t, off));
    const uint32_t scs = lds_u16(t, off + 2 + 2 * g);
    w.sca = (int)(int8_t)(scs & 0xffu);
    w.scb = (int)(int8_t)(scs >> 8);
    uint32_t ql[4], qh[2];
    lds_read_unaligned<4>(t, off + 18 + 16 * g, ql);
    lds_read_unaligned<2>(t, off + 146 + 8 * g, qh);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w.c[i] = (ql[i] & 0x0F0F0F0Fu) | hi2(qh[i & 1], i >> 1);
      w.c[4 + i] = ((ql[i] >> 4) & 0x0F0F0F0Fu) | hi2(qh[(4 + i) & 1], (4 + i) >> 1);
    }
    return w;
  }
  // 16-element partial sums of xq * (q - 32)
  QG_DEV static void pdot(const W& w, const Act& a, int& p0, int& p1) {
    int s0 = 0, s1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0 = dot4((int)w.c[i], a.x[i], s0);
      s1 = dot4((int)w.c[4 + i], a.x[4 + i], s1);
    }
    p0 = s0 - 32 * a.sa;
    p1 = s1 - 32 * a.sb;
  }
  QG_DEV static float fma(const W& w, const Act& a, float acc) {
    int p0, p1;
    pdot(w, a, p0, p1);
    return fmaf(a.dx * w.d, (float)(w.sca * p0 + w.scb * p1), acc);
  }
  QG_DEV static void dots(const W& w, const Act& a, int32_t* out) {
    int p0, p1;
    pdot(w, a, p0, p1);
    out[0] = p0;
    out[1] = p1;
  }
  static constexpr int kDotsPerUnit = 2;
};

template <int FMT> struct FmtOf;
template <> struct FmtOf<kQ4_0> { using T = FmtQ4_0; };
template <> struct FmtOf<kQ8_0> { using T = FmtQ8_0; };
template <> struct FmtOf<kIQ4_NL> { using T = FmtIQ4_NL; };
template <> struct FmtOf<kQ4_K> { using T = FmtQ4_K; };
template <> struct FmtOf<kQ6_K> { using T = FmtQ6_K; };
template <> struct FmtOf<kQ5_K> { using T = FmtQ5_K; };
template <> struct FmtOf<kIQ4_XS> { using T = FmtIQ4_XS; };

}  // namespace qg
