// Row GEMV over packed block-quantized weights, m <= 16 tokens (gfx950).
//
// The weights are read once, in their packed block form, with no fp16 or
// int8 expansion of the matrix; each block is decoded in registers and
// multiplied with int8 activation blocks by 4-way int8 dot products, then
// scaled. K-quant super-blocks apply their scale and min correction terms and
// the non-linear 4-bit format looks its codes up in a 16-entry codebook held
// in registers ("Why expert caching can't save dense models", xhh.club, Q&A
// on computing GGUF blocks without FP16 expansion). The memory-access
// granularity is what decides speed for this bandwidth-bound kernel ("01 ·
// Phase overview: from 2B to 8B to MoE", icman.com.cn, ledger item ㉑).
//
// Kernel structure (one design for all five formats):
//  * A workgroup is 4 waves. At start it stages the quantized activations
//    of all its tokens in LDS, in a layout that makes each lane's 32-element
//    unit a conflict-free 16-byte read: per token, the first 16 codes of
//    every unit, then the last 16 codes of every unit, then (dx, packed
//    16-element sums) per unit.
//  * Each wave then walks "steps": a step is G whole rows (short rows) or one
//    K-segment of one row (long rows) -- a contiguous byte range of the
//    matrix. The wave loads the range with fully coalesced 128-bit loads
//    (lane l takes 16-byte chunks l, l+64, ...) into registers one step
//    ahead, writes it to a wave-private LDS buffer, and decodes from there:
//    blocks of 18, 34 and 210 bytes are not 16-byte aligned, so the LDS hop
//    turns the coalesced byte stream into per-lane block views.
//  * Lane l owns 32-element units l % LPR + LPR * j of row l / LPR within a
//    pass (LPR = lanes per row, 64 when K >= 2048). Each lane keeps fp32
//    partial sums per row; the LPR lanes of a row are summed by a butterfly
//    and one lane stores y. No atomics: results are bitwise reproducible.
#include "common.cuh"
#include "internal.h"

namespace qg {

constexpr int kWavesPerWG = 4;
constexpr int kTileCap = 10240;                 // packed bytes per step (max)
constexpr int kTileBuf = kTileCap + 48;          // + alignment and over-read slack
constexpr int kLoadsPerLane = (kTileCap + 32 + 1023) / 1024;
constexpr int kMaxPasses = 8;                    // row passes per step (M = 1)
constexpr int kLdsLimit = 160 * 1024;

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

// 4 codebook indices (one per byte, 0..15) -> 4 int8 codebook values.
// Entries 0..7 come from {cb1:cb0}, 8..15 from {cb3:cb2}; bit 3 of each
// index then picks between the two candidates with a third byte permute.
QG_DEV uint32_t cb_lookup4(uint32_t idx, const uint32_t* cb) {
  const uint32_t sel = idx & 0x07070707u;
  const uint32_t lo = perm(cb[1], cb[0], sel);
  const uint32_t hi = perm(cb[3], cb[2], sel);
  const uint32_t pick = ((idx >> 1) & 0x04040404u) | 0x03020100u;
  return perm(hi, lo, pick);
}

struct FmtIQ4_NL {
  static constexpr int kUPB = 1, kBB = 18;
  struct W { uint32_t v[8]; float d; };
  QG_DEV static W load(const uint8_t* t, uint32_t off, int, const uint32_t* cb) {
    W w;
    uint32_t q[4];
    w.d = half_bits(lds_u16(t, off));
    lds_read_unaligned<4>(t, off + 2, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w.v[i] = cb_lookup4(q[i] & 0x0F0F0F0Fu, cb);
      w.v[4 + i] = cb_lookup4((q[i] >> 4) & 0x0F0F0F0Fu, cb);
    }
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

// ------------------------------------------------------------ the kernel --

struct GemvGeom {
  int U;          // 32-element units per row
  int LPR, RPP;   // lanes per row, rows per pass
  int P;          // passes per step (rows per step = P * RPP)
  int SU;         // units per step segment (== U when rows are whole)
  int nseg;       // segments per row
  int64_t rb;     // row bytes
  int64_t nrowtiles;
  int act_bytes;  // LDS bytes of staged activations
};

struct GemvArgs {
  GemvProblem p;
  GemvGeom g;
};

template <typename F>
QG_DEV int64_t seg_bytes(int units) { return (int64_t)(units / F::kUPB) * F::kBB; }

template <int FMT, int MT, bool DOTS>
__global__ __launch_bounds__(256) void gemv_kernel(const GemvArgs args) {
  using F = typename FmtOf<FMT>::T;
  constexpr int PM = (MT == 1) ? kMaxPasses : ((32 / MT) < 1 ? 1 : (32 / MT));
  extern __shared__ __align__(16) uint8_t smem[];
  const GemvProblem& p = args.p;
  const GemvGeom& g = args.g;
  const int prob = blockIdx.y;

  // Resolve this problem's matrix, token count and row mapping.
  const uint8_t* W = p.w;
  int mcnt = p.m;
  const int32_t* rows = nullptr;  // grouped mode: slot row of each token
  bool shared = false;
  if (p.tbl) {
    if (prob == p.nprob - 1) {
      W = p.w_shared;
      shared = true;
    } else {
      if (prob >= p.tbl[0]) return;  // whole workgroup leaves before any barrier
      const int32_t* e = p.tbl + 1 + (int64_t)prob * p.tbl_stride;
      W = p.w + (int64_t)e[0] * p.w_stride;
      mcnt = e[1];
      rows = e + 2;
    }
  }
  auto out_row = [&](int t) __attribute__((always_inline)) -> int64_t {
    if (!p.tbl) return t;
    return shared ? (int64_t)t * p.slots + p.slots - 1 : (int64_t)rows[t];
  };

  // ---- stage activations (all tokens) in LDS
  const int U = g.U;
  const int tokb = act_token_bytes(U);
  for (int idx = threadIdx.x; idx < MT * U; idx += blockDim.x) {
    const int t = idx / U, u = idx - t * U;
    uint8_t* tok = smem + t * tokb;
    int4 lo = make_int4(0, 0, 0, 0), hi = make_int4(0, 0, 0, 0);
    float d = 0.0f;
    if (t < mcnt) {
      const int64_t ar = out_row(t) / p.act_div;
      const int4* src = reinterpret_cast<const int4*>(p.xq + ar * p.xs + 32 * u);
      lo = src[0];
      hi = src[1];
      if constexpr (!DOTS) d = p.dx[ar * (p.xs / 32) + u];
    }
    const int ones = 0x01010101;
    int sa = dot4(lo.x, ones, dot4(lo.y, ones, dot4(lo.z, ones, dot4(lo.w, ones, 0))));
    int sb = dot4(hi.x, ones, dot4(hi.y, ones, dot4(hi.z, ones, dot4(hi.w, ones, 0))));
    *reinterpret_cast<int4*>(tok + 16 * u) = lo;
    *reinterpret_cast<int4*>(tok + 16 * U + 16 * u) = hi;
    *reinterpret_cast<int2*>(tok + 32 * U + 8 * u) =
        make_int2(__float_as_int(d), (sa & 0xffff) | (sb << 16));
  }
  __syncthreads();

  const int wid = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  uint8_t* tile = smem + g.act_bytes + wid * kTileBuf;
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerWG;
  const int lam = lane % g.LPR;
  const int rho = lane / g.LPR;
  const int G = g.P * g.RPP;

  // Byte range of step (rt, seg), relative to W.
  auto step_range = [&](int64_t rt, int seg, int64_t& b0, int64_t& b1) __attribute__((always_inline)) {
    const int64_t r0 = rt * G;
    const int64_t nrows = (p.n - r0) < G ? (p.n - r0) : G;
    if (g.nseg == 1) {
      b0 = r0 * g.rb;
      b1 = (r0 + nrows) * g.rb;
    } else {
      const int u0 = seg * g.SU;
      const int su = (U - u0) < g.SU ? (U - u0) : g.SU;
      b0 = r0 * g.rb + seg_bytes<F>(u0);
      b1 = b0 + seg_bytes<F>(su);
    }
  };

  u32x4 buf[kLoadsPerLane];
  auto issue = [&](int64_t rt, int seg) __attribute__((always_inline)) {
    int64_t b0, b1;
    step_range(rt, seg, b0, b1);
    const int64_t a0 = b0 & ~(int64_t)15;
    const int nch = (int)((((b1 + 15) & ~(int64_t)15) - a0) >> 4);
    const u32x4* src = reinterpret_cast<const u32x4*>(W + a0);
#pragma unroll
    for (int i = 0; i < kLoadsPerLane; ++i) {
      const int c = lane + kWave * i;
      if (c < nch) buf[i] = src[c];
    }
  };

  float acc[PM][MT];
#pragma unroll
  for (int a = 0; a < PM; ++a)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[a][t] = 0.0f;

  int64_t rt = (int64_t)blockIdx.x * kWavesPerWG + wid;
  int seg = 0;
  if (rt < g.nrowtiles) issue(rt, seg);

  while (rt < g.nrowtiles) {
    int64_t b0, b1;
    step_range(rt, seg, b0, b1);
    const int64_t a0 = b0 & ~(int64_t)15;
    {
      const int nch = (int)((((b1 + 15) & ~(int64_t)15) - a0) >> 4);
#pragma unroll
      for (int i = 0; i < kLoadsPerLane; ++i) {
        const int c = lane + kWave * i;
        if (c < nch) *reinterpret_cast<u32x4*>(tile + 16 * c) = buf[i];
      }
    }
    // Prefetch the next step of this wave.
    int64_t rt2 = rt;
    int seg2 = seg + 1;
    if (seg2 == g.nseg) { seg2 = 0; rt2 = rt + nwaves; }
    if (rt2 < g.nrowtiles) issue(rt2, seg2);

    // ---- compute this step from LDS
    const int64_t r0 = rt * G;
    const int nrows = (int)((p.n - r0) < G ? (p.n - r0) : G);
    const int u0 = seg * g.SU;
    const int su = (U - u0) < g.SU ? (U - u0) : g.SU;
    const uint32_t base = (uint32_t)(b0 - a0);  // LDS offset of the step's first byte
    for (int j = 0; lam + g.LPR * j < su; ++j) {
      const int ul = lam + g.LPR * j;
      const int ug = u0 + ul;
      // Few tokens: keep every token's unit in registers across the passes;
      // many tokens: re-read it from LDS per row to bound register use.
      constexpr bool kActRegs = MT <= 4;
      Act av[kActRegs ? MT : 1];
      if constexpr (kActRegs) {
#pragma unroll
        for (int t = 0; t < MT; ++t) av[t] = load_act(smem + t * tokb, U, ug);
      }
      const uint32_t uoff = (uint32_t)((ul / F::kUPB) * F::kBB);
      const int sub = ul % F::kUPB;
#pragma unroll
      for (int pp = 0; pp < PM; ++pp) {
        const int rl = pp * g.RPP + rho;
        if (pp < g.P && rl < nrows) {
          const typename F::W wv = F::load(tile, base + (uint32_t)(rl * g.rb) + uoff, sub, p.cb);
          if constexpr (DOTS) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              if (t < mcnt) {
                int32_t* o = p.dots + (out_row(t) * p.n + r0 + rl) * ((int64_t)U * F::kDotsPerUnit) +
                             (int64_t)ug * F::kDotsPerUnit;
                if constexpr (kActRegs) F::dots(wv, av[t], o);
                else F::dots(wv, load_act(smem + t * tokb, U, ug), o);
              }
            }
          } else {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              if (t < mcnt) {  // wave-uniform: skips padded tokens
                if constexpr (kActRegs) acc[pp][t] = F::fma(wv, av[t], acc[pp][t]);
                else acc[pp][t] = F::fma(wv, load_act(smem + t * tokb, U, ug), acc[pp][t]);
              }
            }
          }
        }
      }
    }

    if (!DOTS && seg == g.nseg - 1) {
#pragma unroll
      for (int pp = 0; pp < PM; ++pp) {
        if (pp < g.P) {
          const int rl = pp * g.RPP + rho;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const float v = group_sum(acc[pp][t], g.LPR);
            if (lam == 0 && rl < nrows && t < mcnt) p.y[out_row(t) * p.ldy + r0 + rl] = v;
            acc[pp][t] = 0.0f;
          }
        }
      }
    }
    rt = rt2;
    seg = seg2;
  }
}

// ------------------------------------------------------------- launchers --

int fmt_block_elems(int fmt) {
  switch (fmt) {
    case kQ4_0: case kQ8_0: case kIQ4_NL: return 32;
    case kQ4_K: case kQ6_K: return 256;
    case kF32: return 1;
    default: return 0;
  }
}

int fmt_block_bytes(int fmt) {
  switch (fmt) {
    case kQ4_0: case kIQ4_NL: return 18;
    case kQ8_0: return 34;
    case kQ4_K: return 144;
    case kQ6_K: return 210;
    case kF32: return 4;
    default: return 0;
  }
}

int64_t fmt_row_bytes(int fmt, int64_t k) {
  const int be = fmt_block_elems(fmt);
  if (be <= 0 || k <= 0 || k % be) return -1;
  return k / be * fmt_block_bytes(fmt);
}

static int floor_pow2(int v) {
  int r = 1;
  while (r * 2 <= v) r *= 2;
  return r;
}

static int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
  }
  return cus;
}

// Choose the step geometry for a format, shape and token tile.
static GemvGeom plan_geom(int fmt, int64_t n, int64_t k, int MT) {
  GemvGeom g{};
  const int upb = (fmt == kQ4_K || fmt == kQ6_K) ? 8 : 1;
  const int bb = fmt_block_bytes(fmt);
  g.U = (int)(k / 32);
  g.rb = fmt_row_bytes(fmt, k);
  g.LPR = g.U >= kWave ? kWave : floor_pow2(g.U);
  g.RPP = kWave / g.LPR;
  const int PM = (MT == 1) ? kMaxPasses : ((32 / MT) < 1 ? 1 : (32 / MT));
  if (g.rb * g.RPP <= kTileCap) {
    g.nseg = 1;
    g.SU = g.U;
    int P = (int)(kTileCap / (g.rb * g.RPP));
    if (P > PM) P = PM;
    if (P < 1) P = 1;
    // Keep enough steps to spread the matrix over the whole chip.
    const int64_t want_waves = (int64_t)device_cus() * 4;
    while (P > 1 && (n + (int64_t)P * g.RPP - 1) / ((int64_t)P * g.RPP) < want_waves) P >>= 1;
    g.P = P;
  } else {
    // Long rows: one row per step, split into K-segments of whole
    // super-blocks that are a multiple of 64 units.
    g.P = 1;
    const int64_t unit_bytes_x64 = (int64_t)64 * bb / upb;  // bytes of 64 units
    int su = (int)(kTileCap / unit_bytes_x64) * 64;
    if (su < 64) su = 64;
    g.SU = su;
    g.nseg = (g.U + su - 1) / su;
  }
  const int64_t G = (int64_t)g.P * g.RPP;
  g.nrowtiles = (n + G - 1) / G;
  g.act_bytes = MT * act_token_bytes(g.U);
  return g;
}

template <int FMT, int MT, bool DOTS>
static hipError_t launch_t(const GemvArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.g.act_bytes + (size_t)kWavesPerWG * kTileBuf;
  static bool attr_set = false;  // raise the dynamic-LDS limit once per kernel
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<FMT, MT, DOTS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int64_t wgs = (a.g.nrowtiles + kWavesPerWG - 1) / kWavesPerWG;
  const int64_t cap = (int64_t)device_cus() * 8;
  if (wgs > cap) wgs = cap;
  hipLaunchKernelGGL((gemv_kernel<FMT, MT, DOTS>), dim3((unsigned)wgs, (unsigned)a.p.nprob),
                     dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int FMT, bool DOTS>
static hipError_t launch_mt(const GemvArgs& a, int mt, hipStream_t s) {
  switch (mt) {
    case 1: return launch_t<FMT, 1, DOTS>(a, s);
    case 2: return launch_t<FMT, 2, DOTS>(a, s);
    case 4: return launch_t<FMT, 4, DOTS>(a, s);
    case 8: return launch_t<FMT, 8, DOTS>(a, s);
    default: return launch_t<FMT, 16, DOTS>(a, s);
  }
}

template <bool DOTS>
static hipError_t launch_fmt(int fmt, const GemvArgs& a, int mt, hipStream_t s) {
  switch (fmt) {
    case kQ4_0: return launch_mt<kQ4_0, DOTS>(a, mt, s);
    case kQ8_0: return launch_mt<kQ8_0, DOTS>(a, mt, s);
    case kQ4_K: return launch_mt<kQ4_K, DOTS>(a, mt, s);
    case kQ6_K: return launch_mt<kQ6_K, DOTS>(a, mt, s);
    case kIQ4_NL: return launch_mt<kIQ4_NL, DOTS>(a, mt, s);
    default: return hipErrorInvalidValue;
  }
}

static int token_tile(int m) {
  if (m <= 1) return 1;
  if (m <= 2) return 2;
  if (m <= 4) return 4;
  if (m <= 8) return 8;
  return 16;
}

hipError_t launch_gemv(int fmt, const GemvProblem& p, bool dots_epilogue, hipStream_t s) {
  if (p.m < 1 || p.m > kGemvMaxTokens || p.n < 1) return hipErrorInvalidValue;
  if (p.tbl && p.m > kGemvMaxTokens) return hipErrorInvalidValue;
  int mt = token_tile(p.m);
  GemvArgs a;
  a.p = p;
  a.g = plan_geom(fmt, p.n, p.k, mt);
  // Keep the staged activations within LDS; fall back to smaller token tiles.
  while ((size_t)a.g.act_bytes + (size_t)kWavesPerWG * kTileBuf > (size_t)kLdsLimit && mt > 1) {
    mt >>= 1;
    a.g = plan_geom(fmt, p.n, p.k, mt);
  }
  if ((size_t)a.g.act_bytes + (size_t)kWavesPerWG * kTileBuf > (size_t)kLdsLimit)
    return hipErrorInvalidValue;
  if (p.tbl && mt < p.m) return hipErrorInvalidValue;  // grouped problems cannot be split
  if (mt >= p.m || p.tbl) return dots_epilogue ? launch_fmt<true>(fmt, a, mt, s) : launch_fmt<false>(fmt, a, mt, s);
  // Token chunks of mt.
  for (int t0 = 0; t0 < p.m; t0 += mt) {
    GemvArgs c = a;
    c.p.m = (p.m - t0) < mt ? (p.m - t0) : mt;
    c.p.xq = p.xq + (int64_t)t0 * p.xs;
    if (p.dx) c.p.dx = p.dx + (int64_t)t0 * (p.xs / 32);
    if (p.y) c.p.y = p.y + (int64_t)t0 * p.ldy;
    if (p.dots) c.p.dots = p.dots + (int64_t)t0 * p.n * (p.k / (fmt == kQ6_K ? 16 : 32));
    hipError_t e = dots_epilogue ? launch_fmt<true>(fmt, c, mt, s) : launch_fmt<false>(fmt, c, mt, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qg
