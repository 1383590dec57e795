// 16-bit activation variant of the decode GEMV.
//
// Int8 activation error compounds over a deep MoE stack; the fix recorded in
// "01 · Phase overview: from 2B to 8B to MoE" (icman.com.cn, issue ledger
// item ⑫) was 16-bit activations, a quantization step 256 times finer. Here
// the activation blocks keep their shape (32 elements, one fp32 scale) with
// scale = absmax / 32767 (IEEE fp32 division) and int16 codes rounded half
// away from zero from the IEEE quotient x / scale.
//
// The GEMV is the register-direct single-token Q4_K / Q5_K kernel's layout
// (lane l owns sub-blocks l, l + 64, ... of every row; the super-block header
// and the sub-block's 16 code bytes are aligned 128-bit loads, plus Q5_K's
// 4-byte word of fifth bits) with the int8 dot
// products replaced by v_dot2_i32_i16: each dword of packed 4-bit codes is
// split into four int16 pairs by masks (elements 4i, 4i+2 | 4i+1, 4i+3 |
// 16+4i, 16+4i+2 | 16+4i+1, 16+4i+3) and the activation codes are permuted
// into the same pairs once, when the lane loads them. The sub-block dot
// D = sum x16 * q (|D| <= 32 * 32767 * 31 < 2^25, exact in int32; exact in
// fp32 for Q4_K, |D| < 2^24, and for Q5_K within one rounding of an fp32
// product of the kind the epilogue already makes) then takes the scale and
// min correction as in the int8 path:
// y += dx * (d * sc) * D - dx * (dmin * m) * sum(x16).
#include "common.cuh"
#include "internal.h"
#include "s16.cuh"
#include "s16.h"

namespace qg {

namespace {

constexpr int kWaves16 = 4;
constexpr int kBuf3 = 0x00020000;  // raw buffer resource, gfx9 family

// Eight lanes per block, four elements each (one 128-bit load).
__global__ __launch_bounds__(256) void quant_s16_kernel(const float* __restrict__ x, int16_t* __restrict__ xq,
                                                        float* __restrict__ dx, int32_t* __restrict__ sx,
                                                        int64_t nblocks) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gt >> 3;
  const int part = (int)(gt & 7);
  if (blk >= nblocks) return;  // whole groups of eight lanes leave together
  const float4 v = reinterpret_cast<const float4*>(x)[blk * 8 + part];
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = max8(a);
  const float d = (a > 0.0f) ? a / 32767.0f : 0.0f;
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (d != 0.0f) {
    q0 = code16(v.x, d);
    q1 = code16(v.y, d);
    q2 = code16(v.z, d);
    q3 = code16(v.w, d);
  }
  uint2 packed;
  packed.x = ((uint32_t)q0 & 0xffffu) | ((uint32_t)q1 << 16);
  packed.y = ((uint32_t)q2 & 0xffffu) | ((uint32_t)q3 << 16);
  reinterpret_cast<uint2*>(xq)[blk * 8 + part] = packed;
  int s = q0 + q1 + q2 + q3;
  s = sum4(s);
  s += other_quad(s);
  if (part == 0) {
    dx[blk] = d;
    sx[blk] = s;
  }
}

QG_DEV uint32_t field6(uint32_t hi, uint32_t lo, uint32_t sh) { return __builtin_amdgcn_alignbit(hi, lo, sh) & 63u; }

// FMT: kQ4_K or kQ5_K; JU sub-blocks per lane per row (K = 2048 JU); R rows
// per wave iteration.
template <int FMT, int JU, int R, bool DOTS>
__global__ __launch_bounds__(kWaves16 * 64) void q4k_s16_kernel(const uint8_t* __restrict__ W,
                                                                 const int16_t* __restrict__ xq,
                                                                 const float* __restrict__ dx,
                                                                 const int32_t* __restrict__ sx,
                                                                 float* __restrict__ y, int32_t* __restrict__ dots,
                                                                 int64_t n, int64_t rb) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * kWaves16 + wid;
  const int64_t nw = (int64_t)gridDim.x * kWaves16;
  const int64_t ngroups = (n + R - 1) / R;

  // Activation codes of sub-blocks u = lane + 64 j, as int16 pairs in the
  // order the weight masks produce them.
  uint32_t xa[JU][16];
  float xd[JU];
  int xsum[JU];
#pragma unroll
  for (int j = 0; j < JU; ++j) {
    const int u = lane + 64 * j;
    const int4* p = reinterpret_cast<const int4*>(xq + 32 * u);
    const int4 a0 = p[0], a1 = p[1], a2 = p[2], a3 = p[3];
    const uint32_t w[16] = {(uint32_t)a0.x, (uint32_t)a0.y, (uint32_t)a0.z, (uint32_t)a0.w,
                            (uint32_t)a1.x, (uint32_t)a1.y, (uint32_t)a1.z, (uint32_t)a1.w,
                            (uint32_t)a2.x, (uint32_t)a2.y, (uint32_t)a2.z, (uint32_t)a2.w,
                            (uint32_t)a3.x, (uint32_t)a3.y, (uint32_t)a3.z, (uint32_t)a3.w};  // w[t] = (x[2t], x[2t+1])
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xa[j][4 * i + 0] = perm(w[2 * i + 1], w[2 * i], 0x05040100u);      // x[4i],      x[4i+2]
      xa[j][4 * i + 1] = perm(w[2 * i + 1], w[2 * i], 0x07060302u);      // x[4i+1],    x[4i+3]
      xa[j][4 * i + 2] = perm(w[9 + 2 * i], w[8 + 2 * i], 0x05040100u);  // x[16+4i],   x[16+4i+2]
      xa[j][4 * i + 3] = perm(w[9 + 2 * i], w[8 + 2 * i], 0x07060302u);  // x[16+4i+1], x[16+4i+3]
    }
    xd[j] = DOTS ? 0.0f : dx[u];
    xsum[j] = DOTS ? 0 : sx[u];
  }
  const int g = lane & 7;
  const bool sc_low = g < 6;
  const uint32_t sc_sh = sc_low ? 6 * g : 6 * g - 32;
  const bool m_low = g < 3;
  const uint32_t m_sh = m_low ? 16 + 6 * g : 6 * g - 16;
  constexpr bool Q5 = FMT == kQ5_K;
  constexpr uint32_t BB = Q5 ? 176u : 144u;  // super-block bytes
  constexpr uint32_t QS = Q5 ? 48u : 16u;    // offset of the low code bits
  uint32_t hoff[JU], qoff[JU], xoff[JU];
#pragma unroll
  for (int j = 0; j < JU; ++j) {
    const uint32_t b = (uint32_t)(lane >> 3) + 8u * j;
    hoff[j] = b * BB;
    qoff[j] = b * BB + QS + 16u * g;
    xoff[j] = b * BB + 16u + 4u * g;  // Q5_K: the sub-block's word of fifth bits
  }

  for (int64_t grp = gw; grp < ngroups; grp += nw) {
    const int64_t r0 = grp * R;
    const int64_t rows = (n - r0) < R ? (n - r0) : R;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W + r0 * rb), 0, (int)(rows * rb), kBuf3);
    u32x4 h[R][JU], q[R][JU];
    uint32_t x5[R][JU];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < JU; ++j) {
        h[r][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(hoff[j] + r * rb), 0, 2);
        q[r][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(qoff[j] + r * rb), 0, 2);
        if constexpr (Q5) x5[r][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(xoff[j] + r * rb), 0, 2);
      }
    float accr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < JU; ++j) {
        const uint32_t qv[4] = {q[r][j].x, q[r][j].y, q[r][j].z, q[r][j].w};
        int D = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t w0 = qv[i] & 0x000F000Fu, w1 = (qv[i] >> 8) & 0x000F000Fu;
          uint32_t w2 = (qv[i] >> 4) & 0x000F000Fu, w3 = (qv[i] >> 12) & 0x000F000Fu;
          if constexpr (Q5) {
            // Fifth bit of sub-block element e at bit 8 (e % 4) + e / 4 of the
            // word, moved to bit 4 of its int16 lane: elements 4i, 4i+2 sit at
            // bits i, 16+i; 4i+1, 4i+3 at 8+i, 24+i; 16+4i, 16+4i+2 at 4+i,
            // 20+i; 16+4i+1, 16+4i+3 at 12+i, 28+i.
            const uint32_t f = x5[r][j];
            w0 |= (f << (4 - i)) & 0x00100010u;
            w1 |= (f >> (4 + i)) & 0x00100010u;
            w2 |= (f >> i) & 0x00100010u;
            w3 |= (f >> (8 + i)) & 0x00100010u;
          }
          D = dot2(w0, xa[j][4 * i + 0], D);
          D = dot2(w1, xa[j][4 * i + 1], D);
          D = dot2(w2, xa[j][4 * i + 2], D);
          D = dot2(w3, xa[j][4 * i + 3], D);
        }
        if constexpr (DOTS) {
          if (r < rows) dots[(r0 + r) * (64 * JU) + lane + 64 * j] = D;
          continue;
        }
        const u32x4 hh = h[r][j];
        const float d = half_bits(hh.x & 0xffffu);
        const float dmin = half_bits(hh.x >> 16);
        const uint32_t sc = sc_low ? field6(hh.z, hh.y, sc_sh) : field6(hh.w, hh.z, sc_sh);
        const uint32_t mn = m_low ? field6(hh.w, hh.z, m_sh) : field6(hh.w, hh.w, m_sh);
        acc = fmaf(xd[j] * (d * (float)sc), (float)D, acc);
        acc = fmaf(-(xd[j] * (dmin * (float)mn)), (float)xsum[j], acc);
      }
      accr[r] = acc;
    }
    if constexpr (!DOTS) {
      // Row totals: lane r ends with row r (four rows reduced together).
      float outv;
      if constexpr (R == 4) {
        outv = rows4_wave_sum(accr[0], accr[1], accr[2], accr[3], lane);
      } else {
        outv = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float sum = group_sum(accr[r], 64);
          if (lane == r) outv = sum;
        }
      }
      if (lane < rows) y[r0 + lane] = outv;
    }
  }
}

template <int FMT, int JU, int R, bool DOTS>
hipError_t launch_ju_t(const uint8_t* w, const int16_t* xq, const float* dx, const int32_t* sx, float* y,
                       int32_t* dots, int64_t n, int64_t k, hipStream_t s) {
  auto kern = q4k_s16_kernel<FMT, JU, R, DOTS>;
  const int cus = device_cus();
  const int64_t ngroups = (n + R - 1) / R;
  int64_t waves = (int64_t)cus * 3 * kWaves16;  // three resident workgroups per CU, as the int8 kernel
  if (waves > ngroups) waves = ngroups;
  const int64_t wgs = (waves + kWaves16 - 1) / kWaves16;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kWaves16 * 64), 0, s, w, xq, dx, sx, y, dots, n,
                     fmt_row_bytes(FMT, k));
  return hipGetLastError();
}

template <int FMT, int R, bool DOTS>
hipError_t launch_r(const uint8_t* w, const int16_t* xq, const float* dx, const int32_t* sx, float* y,
                    int32_t* dots, int64_t n, int64_t k, hipStream_t s) {
  switch (k / 2048) {
    case 1: return launch_ju_t<FMT, 1, R, DOTS>(w, xq, dx, sx, y, dots, n, k, s);
    case 2: return launch_ju_t<FMT, 2, R, DOTS>(w, xq, dx, sx, y, dots, n, k, s);
    case 3: return launch_ju_t<FMT, 3, R, DOTS>(w, xq, dx, sx, y, dots, n, k, s);
    default: return launch_ju_t<FMT, 4, R, DOTS>(w, xq, dx, sx, y, dots, n, k, s);
  }
}

template <int FMT>
hipError_t launch_fmt16(const uint8_t* w, const int16_t* xq, const float* dx, const int32_t* sx, float* y,
                        int32_t* dots, int64_t n, int64_t k, hipStream_t s) {
  // Four rows per wave iteration for large matrices, one for small ones.
  if (dots) return n >= 8192 ? launch_r<FMT, 4, true>(w, xq, dx, sx, y, dots, n, k, s)
                             : launch_r<FMT, 1, true>(w, xq, dx, sx, y, dots, n, k, s);
  return n >= 8192 ? launch_r<FMT, 4, false>(w, xq, dx, sx, y, dots, n, k, s)
                   : launch_r<FMT, 1, false>(w, xq, dx, sx, y, dots, n, k, s);
}

}  // namespace

hipError_t launch_quant_s16(const float* x, int16_t* xq, float* dx, int32_t* sx, int64_t nblocks, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  const int64_t threads = nblocks * 8;
  hipLaunchKernelGGL(quant_s16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, xq, dx, sx,
                     nblocks);
  return hipGetLastError();
}

bool s16_gemv_ok(int fmt, int64_t n, int64_t k) {
  return (fmt == kQ4_K || fmt == kQ5_K) && n >= 1 && k % 2048 == 0 && k / 2048 >= 1 && k / 2048 <= 4;
}

hipError_t launch_kquant_s16(int fmt, const uint8_t* w, const int16_t* xq, const float* dx, const int32_t* sx,
                             float* y, int32_t* dots, int64_t n, int64_t k, hipStream_t s) {
  if (!s16_gemv_ok(fmt, n, k)) return hipErrorInvalidValue;
  return fmt == kQ4_K ? launch_fmt16<kQ4_K>(w, xq, dx, sx, y, dots, n, k, s)
                      : launch_fmt16<kQ5_K>(w, xq, dx, sx, y, dots, n, k, s);
}

}  // namespace qg

// ---------------------------------------------------------------------------
// MoE experts on 16-bit activations (the layer where the pages used them).

namespace qg {

namespace {

// Grouped single-token Q4_0 GEMV on 16-bit codes. grid = (workgroups per
// entry, entries); entry e of the grouping table is {expert (-1: shared),
// token count (1), output row}; its activation row is output row / act_div.
// LPR lanes per row (one 18-byte block each, JB blocks per lane): a block is
// read as five aligned dwords around it (its offset is even; rows and
// matrices are multiples of 4 bytes, so the window never passes the
// matrix's end), its 16 code bytes re-aligned with one byte shift when the
// block starts at 2 mod 4. The nibble order is the K-quant sub-block's, so
// the int16 pairing of the Q4_K kernel applies; the -8 offset is the block
// sum: D = sum x16 * q - 8 * sum x16.
template <int LPR, int JB>
__global__ __launch_bounds__(kWaves16 * 64) void q40_s16_grouped_kernel(
    const uint8_t* __restrict__ W, int64_t w_stride, const uint8_t* __restrict__ W_shared,
    const int32_t* __restrict__ tbl, int tbl_stride, const int16_t* __restrict__ xq, const float* __restrict__ dx,
    const int32_t* __restrict__ sx, int64_t xs, int act_div, float* __restrict__ y, int64_t ldy, int64_t n) {
  const int prob = blockIdx.y;
  if (prob >= tbl[0]) return;  // whole workgroup, before any cross-lane step
  const int32_t* ent = tbl + 1 + (int64_t)prob * tbl_stride;
  const uint8_t* Wm = ent[0] < 0 ? W_shared : W + (int64_t)ent[0] * w_stride;
  const int64_t orow = ent[2];
  const int64_t arow = orow / act_div;
  constexpr int U = LPR * JB;       // blocks per row
  constexpr int RPP = 64 / LPR;     // rows per wave pass
  constexpr int RB = U * 18;        // row bytes
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane / LPR, lb = lane % LPR;

  uint32_t xa[JB][16];
  float xd[JB];
  int xsum[JB];
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int b = lb + LPR * j;
    const int4* p = reinterpret_cast<const int4*>(xq + arow * xs + 32 * b);
    const int4 a0 = p[0], a1 = p[1], a2 = p[2], a3 = p[3];
    const uint32_t w[16] = {(uint32_t)a0.x, (uint32_t)a0.y, (uint32_t)a0.z, (uint32_t)a0.w,
                            (uint32_t)a1.x, (uint32_t)a1.y, (uint32_t)a1.z, (uint32_t)a1.w,
                            (uint32_t)a2.x, (uint32_t)a2.y, (uint32_t)a2.z, (uint32_t)a2.w,
                            (uint32_t)a3.x, (uint32_t)a3.y, (uint32_t)a3.z, (uint32_t)a3.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xa[j][4 * i + 0] = perm(w[2 * i + 1], w[2 * i], 0x05040100u);
      xa[j][4 * i + 1] = perm(w[2 * i + 1], w[2 * i], 0x07060302u);
      xa[j][4 * i + 2] = perm(w[9 + 2 * i], w[8 + 2 * i], 0x05040100u);
      xa[j][4 * i + 3] = perm(w[9 + 2 * i], w[8 + 2 * i], 0x07060302u);
    }
    xd[j] = dx[arow * (xs / 32) + b];
    xsum[j] = sx[arow * (xs / 32) + b];
  }
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Wm), 0, (int)(n * RB), kBuf3);
  const int64_t gw = (int64_t)blockIdx.x * kWaves16 + wid;
  const int64_t nw = (int64_t)gridDim.x * kWaves16;
  for (int64_t r0 = gw * RPP; r0 < n; r0 += nw * RPP) {
    const int64_t row = r0 + lr;
    float acc = 0.0f;
    if (row < n) {
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int off = (int)(row * RB) + 18 * (lb + LPR * j);
        const int base = off & ~3;
        uint32_t dw[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) dw[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, base + 4 * i, 0, 2);
        const bool odd = (off & 3) != 0;  // block starts at 2 mod 4
        const float d = half_bits(odd ? (dw[0] >> 16) : (dw[0] & 0xffffu));
        int D = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t q = odd ? dw[i + 1] : alignbyte(dw[i + 1], dw[i], 2);
          D = dot2(q & 0x000F000Fu, xa[j][4 * i + 0], D);
          D = dot2((q >> 8) & 0x000F000Fu, xa[j][4 * i + 1], D);
          D = dot2((q >> 4) & 0x000F000Fu, xa[j][4 * i + 2], D);
          D = dot2((q >> 12) & 0x000F000Fu, xa[j][4 * i + 3], D);
        }
        D -= 8 * xsum[j];
        acc = fmaf(xd[j] * d, (float)D, acc);
      }
    }
    const float sum = group_sum(acc, LPR);
    if (lb == 0 && row < n) y[orow * ldy + row] = sum;
  }
}

// SwiGLU + 16-bit re-quantization of h, eight lanes per 32-element block
// (the stand-alone SwiGLU kernel's layout with the 16-bit rule).
__global__ __launch_bounds__(256) void swiglu_s16_kernel(const float* __restrict__ gu, int64_t gu_ld,
                                                         float* __restrict__ h, int16_t* __restrict__ hq,
                                                         float* __restrict__ hd, int32_t* __restrict__ hs,
                                                         int64_t rows, int64_t inter) {
  const int64_t nbr = inter / 32;
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gt >> 3;
  const int part = (int)(gt & 7);
  if (blk >= rows * nbr) return;  // whole groups of eight lanes leave together
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
  const float d = (a > 0.0f) ? a / 32767.0f : 0.0f;
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (d != 0.0f) {
    q0 = code16(v.x, d);
    q1 = code16(v.y, d);
    q2 = code16(v.z, d);
    q3 = code16(v.w, d);
  }
  uint2 packed;
  packed.x = ((uint32_t)q0 & 0xffffu) | ((uint32_t)q1 << 16);
  packed.y = ((uint32_t)q2 & 0xffffu) | ((uint32_t)q3 << 16);
  *reinterpret_cast<uint2*>(hq + r * inter + col) = packed;
  int s = q0 + q1 + q2 + q3;
  s = sum4(s);
  s += other_quad(s);
  if (part == 0) {
    hd[r * nbr + b] = d;
    hs[r * nbr + b] = s;
  }
}

template <int LPR, int JB>
hipError_t launch_q40g(const S16Grouped& a, hipStream_t s) {
  const int cus = device_cus();
  // Workgroups per entry: enough row passes for every wave, and no more
  // workgroups in all than about four per CU resident at once.
  constexpr int RPP = 64 / LPR;
  int64_t per = ((int64_t)cus * 4 + a.nprob - 1) / a.nprob;
  const int64_t need = (a.n + (int64_t)kWaves16 * RPP - 1) / ((int64_t)kWaves16 * RPP);
  if (per > need) per = need;
  if (per < 1) per = 1;
  hipLaunchKernelGGL((q40_s16_grouped_kernel<LPR, JB>), dim3((unsigned)per, (unsigned)a.nprob),
                     dim3(kWaves16 * 64), 0, s, a.w, a.w_stride, a.w_shared, a.tbl, a.tbl_stride, a.xq, a.dx, a.sx,
                     a.xs, a.act_div, a.y, a.ldy, a.n);
  return hipGetLastError();
}

}  // namespace

bool q40_s16_grouped_ok(int64_t k) { return k == 512 || k == 1024 || k == 2048 || k == 4096; }

hipError_t launch_q40_s16_grouped(const S16Grouped& a, hipStream_t s) {
  if (!q40_s16_grouped_ok(a.k) || a.n < 1 || a.nprob < 1) return hipErrorInvalidValue;
  switch (a.k) {
    case 512: return launch_q40g<16, 1>(a, s);
    case 1024: return launch_q40g<32, 1>(a, s);
    case 2048: return launch_q40g<64, 1>(a, s);
    default: return launch_q40g<64, 2>(a, s);
  }
}

hipError_t launch_swiglu_s16(const float* gu, int64_t gu_ld, float* h, int16_t* hq, float* hd, int32_t* hs,
                             int64_t rows, int64_t inter, hipStream_t s) {
  const int64_t threads = rows * (inter / 32) * 8;
  if (threads <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_s16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, gu, gu_ld, h,
                     hq, hd, hs, rows, inter);
  return hipGetLastError();
}

}  // namespace qg
