// Single-token GEMV over Q4_K, Q5_K and IQ4_XS super-blocks read straight
// into registers.
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
// lane; the 64 lanes of a row are summed in a fixed order (DPP, lane swaps).
//
// IQ4_XS (136-byte super-blocks: d, the sub-scales' high bits, their low
// nibbles, 128 code bytes) has the same sub-block shape: the lane reads the
// 8-byte header and its sub-block's 16 code bytes (both 8-byte aligned),
// maps the codes through the codebook (two byte permutes and an xor per
// four codes, as in the LDS-staged kernel) and adds dx * d * (ls_j - 32) * D.
#include "common.cuh"
#include "formats.cuh"
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
#ifndef QG_Q4K_RFUSED
#define QG_Q4K_RFUSED 2          // the same with the quantizer fused (one workgroup per CU), all formats
#endif
#ifndef QG_IQ4XS_DIRECT
#define QG_IQ4XS_DIRECT 1        // single-token IQ4_XS GEMVs use this kernel too
#endif
#ifndef QG_DIRECT_FUSED_WGS_PER_CU
#define QG_DIRECT_FUSED_WGS_PER_CU 1
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

// Kernel arguments.
struct DirectArgs {
  const uint8_t* w;
  const int8_t* xq;      // quantized activations (unfused)
  const float* dx;
  const float* xf;       // fp32 activations (fused quantization)
  int8_t* xq_out;        // fused: workgroup 0 writes the codes here (optional)
  float* dx_out;
  int32_t* sx_out;
  float* y;
  int32_t* dots;
  int64_t n, rb;
  uint32_t cb[4];        // IQ4_XS: the codebook's byte-permute pools
};

// FMT: kQ4_K or kQ5_K; R rows per iteration; JU sub-blocks per lane per row.
// DOTS: store the exact per-sub-block integer dots D (int32 [n, 64 JU])
// instead of y. FUSEQ: quantize the fp32 activations in the prologue (once
// per workgroup, into LDS) instead of reading codes written by a separate
// launch; NW waves per workgroup.
template <int FMT, int JU, int R, bool DOTS, bool FUSEQ, int NW>
__global__ __launch_bounds__(NW * 64) void kdirect_kernel(const DirectArgs A) {
  const uint8_t* __restrict__ W = A.w;
  float* __restrict__ y = A.y;
  int32_t* __restrict__ dots = A.dots;
  const int64_t n = A.n, rb = A.rb;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * NW + wid;
  const int64_t nw = (int64_t)gridDim.x * NW;
  const int64_t ngroups = (n + R - 1) / R;

  // Activations of this lane's sub-blocks u = lane + 64 j: codes, scale and
  // code sum (filled below, after the first weight loads are issued).
  int xa[JU][8];
  float xd[JU];
  int xsum[JU];

  // Sub-block g = lane % 8 of its super-block. Scale field sc_g sits at bit
  // 6g of the 96-bit stream (header dwords 1..3), min m_g at bit 48 + 6g.
  const int g = lane & 7;
  const bool sc_low = g < 6;     // sc_g within dwords {1, 2}, else {2, 3}
  const uint32_t sc_sh = sc_low ? 6 * g : 6 * g - 32;
  const bool m_low = g < 3;      // m_g within dwords {2, 3}, else dword 3
  const uint32_t m_sh = m_low ? 16 + 6 * g : 6 * g - 16;
  constexpr bool Q5 = FMT == kQ5_K;
  constexpr bool XS = FMT == kIQ4_XS;
  constexpr uint32_t BB = Q5 ? 176u : XS ? 136u : 144u;  // super-block bytes
  constexpr uint32_t QS = Q5 ? 48u : XS ? 8u : 16u;      // offset of the (low) code bits
  uint32_t cbr[4] = {A.cb[0], A.cb[1], A.cb[2], A.cb[3]};
  if constexpr (XS) {
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(cbr[i]));  // pools in VGPRs for the permutes
  }
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
        if constexpr (XS) {
          const auto hv = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(hoff[j] + r * rb), 0, kNonTemporal);
          h[r][j] = u32x4{hv[0], hv[1], 0u, 0u};
        } else {
          h[r][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(hoff[j] + r * rb), 0, kNonTemporal);
        }
        q[r][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(qoff[j] + r * rb), 0, kNonTemporal);
        if constexpr (Q5)
          x5[r][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(xoff[j] + r * rb), 0, kNonTemporal);
      }
  };

  auto consume = [&](const u32x4 (&h)[R][JU], const u32x4 (&q)[R][JU], const uint32_t (&x5)[R][JU],
                     int64_t grp) __attribute__((always_inline)) {
    const int64_t r0 = grp * R;
    float accr[R];
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
          if constexpr (XS) {
            uint32_t vlo, vhi;
            cb_lookup8(qv[i], cbr, vlo, vhi);
            D = dot4((int)vlo, xa[j][i], D);
            D = dot4((int)vhi, xa[j][4 + i], D);
            continue;
          }
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
        if constexpr (XS) {
          // 6-bit sub-scale: low nibble g of scales_l, high bits 2g of scales_h
          const uint32_t ls = ((hh.y >> (4 * g)) & 0xFu) | (((hh.x >> (16 + 2 * g)) & 3u) << 4);
          acc = fmaf(xd[j] * (half_bits(hh.x & 0xffffu) * (float)((int)ls - 32)), (float)D, acc);
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
      accr[r] = acc;
    }
    if constexpr (!DOTS) {
      // Row totals: lane r ends with row r.
      float outv;
      if constexpr (R == 4) {
        outv = rows4_wave_sum(accr[0], accr[1], accr[2], accr[3], lane);
      } else if constexpr (R == 2) {
        outv = rows2_wave_sum(accr[0], accr[1], lane);
      } else {
        outv = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float sum = group_sum(accr[r], 64);
          if (lane == r) outv = sum;
        }
      }
      const int64_t rows = (n - r0) < R ? (n - r0) : R;
      if (lane < rows) y[r0 + lane] = outv;
    }
  };

  // One row group in flight per wave; other resident waves cover the wait.
  // With the quantizer fused and groups of several rows, this thread's fp32 x
  // is requested first and the first row group right after it: loads return
  // in issue order, so x is quantized while the weights are still in flight
  // (measured: 12288 rows 9.8 -> 8.9 us, 24576 rows 13.6 -> 12.6 us). With one
  // row per group (fewer than 8192 rows) the row goes first (4096 rows: 4.9
  // against 5.3 us the other way round).
  constexpr bool kXFirst = FUSEQ && R > 1;
  constexpr int kXPre = (64 * JU * 8 + NW * 64 - 1) / (NW * 64);  // x tasks per thread
  float4 xpre[FUSEQ ? kXPre : 1];
  auto load_x = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < kXPre; ++r) {
      const int i = threadIdx.x + r * NW * 64;
      xpre[r] = i < 64 * JU * 8 ? reinterpret_cast<const float4*>(A.xf)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if constexpr (kXFirst) load_x();
  u32x4 hA[R][JU], qA[R][JU];
  uint32_t xA[R][JU];
  load(hA, qA, xA, gw);
  if constexpr (FUSEQ && !kXFirst) load_x();

  if constexpr (FUSEQ) {
    // Quantize x once per workgroup into LDS: eight lanes per 32-element
    // block, the activation quantizer's arithmetic; workgroup 0 also stores
    // the codes for the caller.
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int U = 64 * JU;
    uint32_t* s_codes = reinterpret_cast<uint32_t*>(smem);            // [U][8] dwords
    float* s_dx = reinterpret_cast<float*>(smem + U * 32);             // [U]
    int* s_sum = reinterpret_cast<int*>(smem + U * 36);                // [U]
    const bool wb = A.xq_out && blockIdx.x == 0;
#pragma unroll
    for (int r = 0; r < kXPre; ++r) {
      const int i = threadIdx.x + r * NW * 64;
      if (i >= U * 8) break;  // whole 8-lane groups in or out
      const float4 v = xpre[r];
      const int u = i >> 3, part = i & 7;
      const float a = max8(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
      const float d = (a > 0.0f) ? a / 127.0f : 0.0f;
      int sm;
      const uint32_t packed = q8_pack4(v, d, sm);
      sm = sum4(sm);
      sm += other_quad(sm);
      s_codes[i] = packed;
      if (part == 0) {
        s_dx[u] = d;
        s_sum[u] = sm;
      }
      if (wb) {
        reinterpret_cast<uint32_t*>(A.xq_out)[i] = packed;
        if (part == 0) {
          A.dx_out[u] = d;
          if (A.sx_out) A.sx_out[u] = sm;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JU; ++j) {
      const int u = lane + 64 * j;
      const int4 lo = *reinterpret_cast<const int4*>(s_codes + 8 * u);
      const int4 hi = *reinterpret_cast<const int4*>(s_codes + 8 * u + 4);
      xa[j][0] = lo.x; xa[j][1] = lo.y; xa[j][2] = lo.z; xa[j][3] = lo.w;
      xa[j][4] = hi.x; xa[j][5] = hi.y; xa[j][6] = hi.z; xa[j][7] = hi.w;
      xd[j] = s_dx[u];
      xsum[j] = s_sum[u];
    }
  } else {
#pragma unroll
    for (int j = 0; j < JU; ++j) {
      const int u = lane + 64 * j;
      const int4 lo = reinterpret_cast<const int4*>(A.xq)[2 * u];
      const int4 hi = reinterpret_cast<const int4*>(A.xq)[2 * u + 1];
      xa[j][0] = lo.x; xa[j][1] = lo.y; xa[j][2] = lo.z; xa[j][3] = lo.w;
      xa[j][4] = hi.x; xa[j][5] = hi.y; xa[j][6] = hi.z; xa[j][7] = hi.w;
      xd[j] = DOTS ? 0.0f : A.dx[u];
      int sm = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) sm = dot4(xa[j][i], 0x01010101, sm);
      xsum[j] = sm;
    }
  }

  for (int64_t grp = gw; grp < ngroups; grp += nw) {
    consume(hA, qA, xA, grp);
    if (grp + nw < ngroups) load(hA, qA, xA, grp + nw);
  }
}

template <int FMT, int JU, int R, bool DOTS, bool FUSEQ, int NW>
hipError_t launch_t(const GemvProblem& p, hipStream_t s) {
  auto kern = kdirect_kernel<FMT, JU, R, DOTS, FUSEQ, NW>;
  const size_t lds = FUSEQ ? (size_t)64 * JU * 40 : 0;
  int nb = 0, cus = 0;  // resident workgroups per CU (cached occupancy query), compute units
  hipError_t qe = kernel_residency(reinterpret_cast<const void*>(kern), NW * 64, lds, false, &nb, &cus);
  if (qe != hipSuccess) return qe;
  const int cap = FUSEQ ? QG_DIRECT_FUSED_WGS_PER_CU : QG_DIRECT_WGS_PER_CU;
  const int per_cu = cap > 0 && cap < nb ? cap : nb;
  const int64_t ngroups = (p.n + R - 1) / R;
  int64_t waves = (int64_t)cus * per_cu * NW;
  if (waves > ngroups) waves = ngroups;
  const int64_t wgs = (waves + NW - 1) / NW;
  DirectArgs a;
  a.w = p.w;
  a.xq = p.xq;
  a.dx = p.dx;
  a.xf = p.xf;
  a.xq_out = p.xq_out;
  a.dx_out = p.dx_out;
  a.sx_out = p.sx_out;
  a.y = p.y;
  a.dots = p.dots;
  a.n = p.n;
  a.rb = fmt_row_bytes(FMT, p.k);
  for (int i = 0; i < 4; ++i) a.cb[i] = p.cb[i];
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

}  // namespace


bool kdirect_ok(int fmt, const GemvProblem& p, bool dots) {
  // fused quantization: one token, K up to 4096 (64 x 2 sub-blocks per lane)
  const bool acts = p.xf ? (!dots && p.k <= 4096 && (!p.xq_out || p.dx_out)) : (p.xq != nullptr);
  return (fmt == kQ4_K || fmt == kQ5_K || (fmt == kIQ4_XS && QG_IQ4XS_DIRECT)) && p.m == 1 && !p.tbl && acts &&
         (dots ? p.dots != nullptr : ((p.xf || p.dx) && p.y)) && p.k % 2048 == 0 && p.k / 2048 >= 1 &&
         p.k / 2048 <= 4 && p.n >= 1;
}

// Waves per workgroup for the fused kernel (one workgroup per CU): the
// count that gives every wave the fewest row groups, then the one that
// keeps the most CUs busy (12 waves: 3072 on 256 CUs, so 12288 and 24576
// rows in groups of four divide evenly; 16 waves: 4096 single rows).
static int fused_waves(int64_t ngroups) {
  const int64_t cus = device_cus();
  int best = 16;
  int64_t best_gpw = 0, best_wgs = 0;
  for (int nw : {16, 12}) {
    const int64_t waves = cus * nw;
    const int64_t gpw = (ngroups + waves - 1) / waves;
    int64_t wgs = (ngroups + gpw * nw - 1) / (gpw * nw);
    if (wgs > cus) wgs = cus;
    if (best_gpw == 0 || gpw < best_gpw || (gpw == best_gpw && wgs > best_wgs)) {
      best = nw;
      best_gpw = gpw;
      best_wgs = wgs;
    }
  }
  return best;
}

template <int FMT, int R, bool DOTS, bool FUSEQ>
static hipError_t launch_ju(const GemvProblem& p, hipStream_t s) {
  if constexpr (FUSEQ) {
    const bool w12 = fused_waves((p.n + R - 1) / R) == 12;
    if (p.k == 2048) return w12 ? launch_t<FMT, 1, R, DOTS, true, 12>(p, s) : launch_t<FMT, 1, R, DOTS, true, 16>(p, s);
    return w12 ? launch_t<FMT, 2, R, DOTS, true, 12>(p, s) : launch_t<FMT, 2, R, DOTS, true, 16>(p, s);
  } else {
    switch (p.k / 2048) {
      case 1: return launch_t<FMT, 1, R, DOTS, false, kDirectWaves>(p, s);
      case 2: return launch_t<FMT, 2, R, DOTS, false, kDirectWaves>(p, s);
      case 3: return launch_t<FMT, 3, R, DOTS, false, kDirectWaves>(p, s);
      default: return launch_t<FMT, 4, R, DOTS, false, kDirectWaves>(p, s);
    }
  }
}

template <int FMT>
static hipError_t launch_fmt(const GemvProblem& p, bool dots, hipStream_t s) {
  // Rows per wave iteration, measured on MI355X (Q4_K): four rows (more
  // bytes in flight per wave) once there are enough rows to still give every
  // CU several waves, one row for smaller matrices (more waves). With the
  // quantizer fused (12 or 16 waves, one workgroup per CU) two rows, for
  // every format: at 12288 rows, groups of four left each wave a single
  // group and nothing to overlap its load with (Q4_K 9.1 -> 7.85 us per
  // call; 24576 rows unchanged).
  constexpr int RB = FMT == kQ5_K ? QG_Q5K_RBIG : QG_Q4K_RBIG;
  constexpr int RF = QG_Q4K_RFUSED;
  if (dots) return p.n >= 8192 ? launch_ju<FMT, RB, true, false>(p, s) : launch_ju<FMT, 1, true, false>(p, s);
  if (p.xf) return p.n >= 8192 ? launch_ju<FMT, RF, false, true>(p, s) : launch_ju<FMT, 1, false, true>(p, s);
  return p.n >= 8192 ? launch_ju<FMT, RB, false, false>(p, s) : launch_ju<FMT, 1, false, false>(p, s);
}

hipError_t launch_kdirect(int fmt, const GemvProblem& p, bool dots, hipStream_t s) {
  if (!kdirect_ok(fmt, p, dots)) return hipErrorInvalidValue;
  if (fmt == kIQ4_XS) return launch_fmt<kIQ4_XS>(p, dots, s);
  return fmt == kQ4_K ? launch_fmt<kQ4_K>(p, dots, s) : launch_fmt<kQ5_K>(p, dots, s);
}

}  // namespace qg
