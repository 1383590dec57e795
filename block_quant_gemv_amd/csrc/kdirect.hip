// Single-token GEMV over Q4_K and Q5_K super-blocks read straight into
// registers.
//
// Both super-blocks (144 and 176 bytes) are multiples of 16, so every field a
// lane needs -- the 16-byte header (d, dmin, the twelve bytes of 6-bit scales
// and mins), the 16 bytes of one 32-element sub-block's low code bits and,
// for Q5_K, the sub-block's 4-byte word of fifth bits -- is an aligned load.
// Lane l of a wave owns sub-blocks l, l + 64, ... of every row (K = 2048 *
// JU), so the eight lanes of one super-block read its header (the same 16
// bytes) and its eight code chunks (128 contiguous bytes, plus 32 contiguous
// bytes of fifth bits): the wave covers whole super-blocks, every byte once. The weights go from HBM to
// registers with no LDS hop, and the quantized activations of the lane's
// sub-blocks stay in registers for the whole kernel, so the main loop uses
// no LDS at all. This is the K-quant in-register decode with scale and min
// correction terms ("Why expert caching can't save dense models", xhh.club,
// Q&A on computing GGUF blocks without FP16 expansion).
//
// Per (row, sub-block j of super-block b): D = sum xq * q over the 32 codes
// (q in 0..15, or 0..31 for Q5_K) and s = sum xq (the activation block sum), then
// y += dx * (d * sc_j) * D - dx * (dmin * m_j) * s, accumulated in fp32 per
// lane; the 64 lanes of a row are summed in a fixed order (DPP, readlane).
#include "common.cuh"
#include "internal.h"

#ifndef QG_DIRECT_WGS_PER_CU
#define QG_DIRECT_WGS_PER_CU 3   // cap on resident workgroups per CU (measured: 3 beats 6)
#endif
#ifndef QG_Q4K_RBIG
#define QG_Q4K_RBIG 4            // rows per wave iteration for large Q4_K matrices
#endif
#ifndef QG_Q5K_RBIG
#define QG_Q5K_RBIG 4            // rows per wave iteration for large Q5_K matrices
#endif
#ifndef QG_Q4K_DIRECT_PF
#define QG_Q4K_DIRECT_PF 1   // row groups in flight per wave (1 or 2)
#endif

namespace qg {

namespace {

constexpr int kDirectWaves = 4;             // waves per workgroup (independent)
constexpr int kBufDword3 = 0x00020000;      // raw buffer resource, gfx9 family
constexpr int kNonTemporal = 2;             // weights are read once

// 6-bit field starting at bit `sh` of the 64-bit value {hi:lo} (sh < 32).
QG_DEV uint32_t field6(uint32_t hi, uint32_t lo, uint32_t sh) {
  return __builtin_amdgcn_alignbit(hi, lo, sh) & 63u;
}

// FMT: kQ4_K or kQ5_K; R rows per iteration; JU sub-blocks per lane per row.
// DOTS: store the exact per-sub-block integer dots D (int32 [n, 64 JU])
// instead of y.
template <int FMT, int JU, int R, bool DOTS>
__global__ __launch_bounds__(kDirectWaves * 64) void kdirect_kernel(const uint8_t* __restrict__ W,
                                                                     const int8_t* __restrict__ xq,
                                                                     const float* __restrict__ dx,
                                                                     float* __restrict__ y,
                                                                     int32_t* __restrict__ dots, int64_t n,
                                                                     int64_t rb) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * kDirectWaves + wid;
  const int64_t nw = (int64_t)gridDim.x * kDirectWaves;
  const int64_t ngroups = (n + R - 1) / R;

  // Activations of this lane's sub-blocks u = lane + 64 j: codes, scale and
  // code sum.
  int xa[JU][8];
  float xd[JU];
  int xsum[JU];
#pragma unroll
  for (int j = 0; j < JU; ++j) {
    const int u = lane + 64 * j;
    const int4 lo = reinterpret_cast<const int4*>(xq)[2 * u];
    const int4 hi = reinterpret_cast<const int4*>(xq)[2 * u + 1];
    xa[j][0] = lo.x; xa[j][1] = lo.y; xa[j][2] = lo.z; xa[j][3] = lo.w;
    xa[j][4] = hi.x; xa[j][5] = hi.y; xa[j][6] = hi.z; xa[j][7] = hi.w;
    xd[j] = DOTS ? 0.0f : dx[u];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot4(xa[j][i], 0x01010101, s);
    xsum[j] = s;
  }
  // Sub-block g = lane % 8 of its super-block. Scale field sc_g sits at bit
  // 6g of the 96-bit stream (header dwords 1..3), min m_g at bit 48 + 6g.
  const int g = lane & 7;
  const bool sc_low = g < 6;     // sc_g within dwords {1, 2}, else {2, 3}
  const uint32_t sc_sh = sc_low ? 6 * g : 6 * g - 32;
  const bool m_low = g < 3;      // m_g within dwords {2, 3}, else dword 3
  const uint32_t m_sh = m_low ? 16 + 6 * g : 6 * g - 16;
  constexpr bool Q5 = FMT == kQ5_K;
  constexpr uint32_t BB = Q5 ? 176u : 144u;     // super-block bytes
  constexpr uint32_t QS = Q5 ? 48u : 16u;       // offset of the low code bits
  uint32_t hoff[JU], qoff[JU], xoff[JU];
#pragma unroll
  for (int j = 0; j < JU; ++j) {
    const uint32_t b = (uint32_t)(lane >> 3) + 8u * j;  // super-block of sub-block lane + 64 j
    hoff[j] = b * BB;
    qoff[j] = b * BB + QS + 16u * g;
    xoff[j] = b * BB + 16u + 4u * g;                    // Q5_K: the sub-block's fifth bits
  }

  // Loads of one row group through a buffer resource spanning exactly its
  // rows: a group past the end reads zeros without touching memory.
  auto load = [&](u32x4 (&h)[R][JU], u32x4 (&q)[R][JU], uint32_t (&x5)[R][JU], int64_t grp)
                  __attribute__((always_inline)) {
    const int64_t r0 = grp * R;
    const int64_t rows = grp < ngroups ? ((n - r0) < R ? (n - r0) : R) : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W + (rows > 0 ? r0 * rb : 0)), 0, (int)(rows * rb), kBufDword3);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < JU; ++j) {
        h[r][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(hoff[j] + r * rb), 0, kNonTemporal);
        q[r][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(qoff[j] + r * rb), 0, kNonTemporal);
        if constexpr (Q5)
          x5[r][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(xoff[j] + r * rb), 0, kNonTemporal);
      }
  };

  auto consume = [&](const u32x4 (&h)[R][JU], const u32x4 (&q)[R][JU], const uint32_t (&x5)[R][JU],
                     int64_t grp) __attribute__((always_inline)) {
    const int64_t r0 = grp * R;
    float outv = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < JU; ++j) {
        const u32x4 hh = h[r][j];
        const uint32_t qv[4] = {q[r][j].x, q[r][j].y, q[r][j].z, q[r][j].w};
        int D = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t lo = qv[i] & 0x0F0F0F0Fu, hi = (qv[i] >> 4) & 0x0F0F0F0Fu;
          if constexpr (Q5) {
            // fifth bit of sub-block element e at bit 8 (e % 4) + e / 4 of
            // the word: bit i of each byte for codes 4i.., bit 4 + i for 16 + 4i..
            lo |= (x5[r][j] << (4 - i)) & 0x10101010u;
            hi |= (x5[r][j] >> i) & 0x10101010u;
          }
          D = dot4((int)lo, xa[j][i], D);
          D = dot4((int)hi, xa[j][4 + i], D);
        }
        if constexpr (DOTS) {
          if (r0 + r < n) dots[(r0 + r) * (64 * JU) + lane + 64 * j] = D;
          continue;
        }
        const float d = half_bits(hh.x & 0xffffu);
        const float dmin = half_bits(hh.x >> 16);
        const uint32_t sc = sc_low ? field6(hh.z, hh.y, sc_sh) : field6(hh.w, hh.z, sc_sh);
        const uint32_t mn = m_low ? field6(hh.w, hh.z, m_sh) : field6(hh.w, hh.w, m_sh);
        const float dsc = d * (float)sc;
        const float dmm = dmin * (float)mn;
        acc = fmaf(xd[j] * dsc, (float)D, acc);
        acc = fmaf(-(xd[j] * dmm), (float)xsum[j], acc);
      }
      if constexpr (!DOTS) {
        const float sum = group_sum(acc, 64);
        if (lane == r) outv = sum;
      }
    }
    if constexpr (!DOTS) {
      const int64_t rows = (n - r0) < R ? (n - r0) : R;
      if (lane < rows) y[r0 + lane] = outv;
    }
  };

#if QG_Q4K_DIRECT_PF > 1
  // Two row groups in flight per wave: A holds group grp, B the next one;
  // each buffer is refilled with the group two ahead once consumed.
  u32x4 hA[R][JU], qA[R][JU], hB[R][JU], qB[R][JU];
  uint32_t xA[R][JU], xB[R][JU];
  load(hA, qA, xA, gw);
  load(hB, qB, xB, gw + nw);
  for (int64_t grp = gw; grp < ngroups; grp += 2 * nw) {
    consume(hA, qA, xA, grp);
    load(hA, qA, xA, grp + 2 * nw);
    if (grp + nw >= ngroups) break;
    consume(hB, qB, xB, grp + nw);
    load(hB, qB, xB, grp + 3 * nw);
  }
#else
  // One row group in flight per wave; other resident waves cover the wait.
  u32x4 hA[R][JU], qA[R][JU];
  uint32_t xA[R][JU];
  for (int64_t grp = gw; grp < ngroups; grp += nw) {
    load(hA, qA, xA, grp);
    consume(hA, qA, xA, grp);
  }
#endif
}

template <int FMT, int JU, int R, bool DOTS>
hipError_t launch_t(const GemvProblem& p, hipStream_t s) {
  auto kern = kdirect_kernel<FMT, JU, R, DOTS>;
  int nb = 0, cus = 0;  // resident workgroups per CU (cached occupancy query), compute units
  hipError_t qe = kernel_residency(reinterpret_cast<const void*>(kern), kDirectWaves * 64, 0, false, &nb, &cus);
  if (qe != hipSuccess) return qe;
  const int per_cu = QG_DIRECT_WGS_PER_CU > 0 && QG_DIRECT_WGS_PER_CU < nb ? QG_DIRECT_WGS_PER_CU : nb;
  const int64_t ngroups = (p.n + R - 1) / R;
  int64_t waves = (int64_t)cus * per_cu * kDirectWaves;
  if (waves > ngroups) waves = ngroups;
  const int64_t wgs = (waves + kDirectWaves - 1) / kDirectWaves;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kDirectWaves * 64), 0, s, p.w, p.xq, p.dx, p.y, p.dots,
                     p.n, fmt_row_bytes(FMT, p.k));
  return hipGetLastError();
}

}  // namespace


bool kdirect_ok(int fmt, const GemvProblem& p, bool dots) {
  return (fmt == kQ4_K || fmt == kQ5_K) && p.m == 1 && !p.tbl && !p.xf && p.xq && (dots ? p.dots != nullptr : (p.dx && p.y)) &&
         p.k % 2048 == 0 && p.k / 2048 >= 1 && p.k / 2048 <= 4 && p.n >= 1;
}

template <int FMT, int R, bool DOTS>
static hipError_t launch_ju(const GemvProblem& p, hipStream_t s) {
  switch (p.k / 2048) {
    case 1: return launch_t<FMT, 1, R, DOTS>(p, s);
    case 2: return launch_t<FMT, 2, R, DOTS>(p, s);
    case 3: return launch_t<FMT, 3, R, DOTS>(p, s);
    default: return launch_t<FMT, 4, R, DOTS>(p, s);
  }
}

template <int FMT>
static hipError_t launch_fmt(const GemvProblem& p, bool dots, hipStream_t s) {
  // Rows per wave iteration, measured on MI355X (Q4_K): four rows (more
  // bytes in flight per wave) once there are enough rows to still give every
  // CU several waves, one row for smaller matrices (more waves).
  constexpr int RB = FMT == kQ5_K ? QG_Q5K_RBIG : QG_Q4K_RBIG;
  if (p.n >= 8192) return dots ? launch_ju<FMT, RB, true>(p, s) : launch_ju<FMT, RB, false>(p, s);
  return dots ? launch_ju<FMT, 1, true>(p, s) : launch_ju<FMT, 1, false>(p, s);
}

hipError_t launch_kdirect(int fmt, const GemvProblem& p, bool dots, hipStream_t s) {
  if (!kdirect_ok(fmt, p, dots)) return hipErrorInvalidValue;
  return fmt == kQ4_K ? launch_fmt<kQ4_K>(p, dots, s) : launch_fmt<kQ5_K>(p, dots, s);
}

}  // namespace qg
