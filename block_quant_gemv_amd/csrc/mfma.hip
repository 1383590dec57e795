// Batched (9..32 tokens per launch tile) GEMM over packed Q4_K / Q6_K
// weights with int8 MFMA, gfx950.
//
// With 32 tokens the work is a real dense contraction: the vector int8 dot
// products of the decode GEMV would make the VALU the bottleneck, so the
// integer block dots run on the matrix cores instead (the prefill/batched
// case of "01 · Phase overview: from 2B to 8B to MoE", icman.com.cn, section
// 九: at batch 32 the dp4a path was exhausted and matrix cores were needed).
// Every MFMA stays inside one scale group -- a 32-element Q4_K sub-block (two
// K=16 MFMAs) or a 16-element Q6_K sub-block (one) -- because each group has
// its own scale (and min), applied in fp32 after the integer product.
//
// v_mfma_i32_32x32x16_i8, D[m][n] += sum_k A[m][k] B[k][n]:
//   A (32 x 16): lane l holds A[l % 32][8 (l / 32) .. +7]   (m = token)
//   B (16 x 32): lane l holds B[8 (l / 32) .. +7][l % 32]   (n = weight row)
//   D (32 x 32): lane l holds D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32], i < 16
// so each lane owns one weight row (its scale fields are per-lane values)
// and 16 tokens. The k order inside a group is free as long as A and B use
// the same one; it is chosen so that each lane's operands are contiguous.
//
// Work split: a wave computes 32 rows x 32 tokens over one K-split of whole
// super-blocks and writes fp32 partial sums; a second kernel adds the
// splits in a fixed order (no atomics, bitwise reproducible).
#include "common.cuh"
#include "internal.h"
#include "mfma.h"

namespace qg {

typedef int v16i __attribute__((ext_vector_type(16)));

#ifndef QG_MFMA_UNROLL
#define QG_MFMA_UNROLL 2   // scale groups of a super-block decoded together
#endif

constexpr int kMT = 32;        // token tile
constexpr int kRowsPerWave = 32;
constexpr int kWaves = 4;      // waves per workgroup: 4 consecutive row tiles, same split

QG_DEV long pack2(uint32_t lo, uint32_t hi) { return (long)(((uint64_t)hi << 32) | lo); }

// Per split: dx and dx * (block sum) of all 32 tokens for the split's
// 32-element blocks, staged in LDS as [block][token].
struct SplitAct {
  float* dx;   // [nblk][32]
  float* c;    // [nblk][32]
};

QG_DEV void stage_split_act(float* lds, const float* dx, const int32_t* sx, int m, int64_t kblocks,
                            int blk0, int nblk) {
  for (int i = threadIdx.x; i < nblk * kMT; i += blockDim.x) {
    const int b = i / kMT, t = i % kMT;
    float d = 0.0f, c = 0.0f;
    if (t < m) {
      d = dx[(int64_t)t * kblocks + blk0 + b];
      c = d * (float)sx[(int64_t)t * kblocks + blk0 + b];
    }
    lds[i] = d;
    lds[nblk * kMT + i] = c;
  }
}

// Q4_K codes of one 16-byte qs chunk: low nibbles (lane group 0) or high
// nibbles (lane group 1), as two 8-byte MFMA operands.
QG_DEV void q4k_operands(const u32x4 q, int g, long& b0, long& b1) {
  const int sh = g ? 4 : 0;
  b0 = pack2((q.x >> sh) & 0x0F0F0F0Fu, (q.y >> sh) & 0x0F0F0F0Fu);
  b1 = pack2((q.z >> sh) & 0x0F0F0F0Fu, (q.w >> sh) & 0x0F0F0F0Fu);
}

// q - 32 for four 6-bit codes q in 0..63, one per byte, as signed int8:
// (q | 0x80) - 0x20 never borrows across bytes, and xor 0x80 recentres.
QG_DEV uint32_t minus32(uint32_t q) { return ((q | 0x80808080u) - 0x20202020u) ^ 0x80808080u; }

template <int FMT, bool DOTS>
__global__ __launch_bounds__(kWaves * 64) void gemm32_kernel(const uint8_t* __restrict__ W,
                                                             const int8_t* __restrict__ xq,
                                                             const float* __restrict__ dx,
                                                             const int32_t* __restrict__ sx,
                                                             float* __restrict__ partials,
                                                             int32_t* __restrict__ dots, int64_t n_rows,
                                                             int64_t k, int m, int splits, int sb_per_split) {
  extern __shared__ __align__(16) float sact[];
  constexpr int BB = FMT == kQ4_K ? 144 : 210;
  const int64_t rb = (k / 256) * BB;
  const int64_t kblocks = k / 32;
  const int nsb_total = (int)(k / 256);
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, col = lane & 31;
  const int split = blockIdx.y;
  const int sb0 = split * sb_per_split;
  int sb1 = sb0 + sb_per_split;
  if (sb1 > nsb_total) sb1 = nsb_total;
  const int nblk = (sb1 - sb0) * 8;  // 32-element blocks in this split

  if constexpr (!DOTS) stage_split_act(sact, dx, sx, m, kblocks, sb0 * 8, nblk);
  __syncthreads();

  const int64_t row0 = ((int64_t)blockIdx.x * kWaves + wid) * kRowsPerWave;
  if (row0 >= n_rows) return;  // after the only barrier
  const int64_t n = row0 + col;
  const int64_t nc = n < n_rows ? n : n_rows - 1;  // ragged last tile: re-read a valid row
  const uint8_t* wrow = W + nc * rb;
  const int t = col;                                 // A-operand token of this lane
  const int8_t* xrow = xq + (int64_t)(t < m ? t : 0) * k;
  const bool tok_ok = t < m;

  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

  for (int sb = sb0; sb < sb1; ++sb) {
    const uint8_t* blk = wrow + (int64_t)sb * BB;
    const int8_t* xs = xrow + (int64_t)sb * 256;
    float accs[16], accm[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { accs[i] = 0.0f; accm[i] = 0.0f; }
    float d, dmin = 0.0f;
    if constexpr (FMT == kQ4_K) {
      const u32x4 h = *reinterpret_cast<const u32x4*>(blk);
      d = half_bits(h.x & 0xffffu);
      dmin = half_bits(h.x >> 16);
      const uint64_t s_lo = (uint64_t)h.y | ((uint64_t)h.z << 32);
      const uint64_t s_hi = (uint64_t)h.z | ((uint64_t)h.w << 32);
#pragma unroll QG_MFMA_UNROLL
      for (int j = 0; j < 8; ++j) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(blk + 16 + 16 * j);
        u32x4 a = {0u, 0u, 0u, 0u};
        if (tok_ok) a = *reinterpret_cast<const u32x4*>(xs + 32 * j + 16 * g);
        long b0, b1;
        q4k_operands(q, g, b0, b1);
        v16i D = {0};
        D = __builtin_amdgcn_mfma_i32_32x32x16_i8(pack2(a.x, a.y), b0, D, 0, 0, 0);
        D = __builtin_amdgcn_mfma_i32_32x32x16_i8(pack2(a.z, a.w), b1, D, 0, 0, 0);
        if constexpr (DOTS) {
          if (n < n_rows) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int tt = 8 * (i >> 2) + 4 * g + (i & 3);
              if (tt < m) dots[((int64_t)tt * n_rows + n) * kblocks + sb * 8 + j] = D[i];
            }
          }
        } else {
          const int sc = (int)((s_lo >> (6 * j)) & 63u);
          const float mn = (float)((s_hi >> (16 + 6 * j)) & 63u);
          const int bl = (sb - sb0) * 8 + j;
          const float4* dxv = reinterpret_cast<const float4*>(sact + bl * kMT);
          const float4* cv = reinterpret_cast<const float4*>(sact + nblk * kMT + bl * kMT);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const float4 dd = dxv[2 * a4 + g];   // tokens 8 a4 + 4 g .. +3
            const float4 cc = cv[2 * a4 + g];
            const float dl[4] = {dd.x, dd.y, dd.z, dd.w};
            const float cl[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * a4 + r;
              accs[i] = fmaf(dl[r], (float)(D[i] * sc), accs[i]);
              accm[i] = fmaf(cl[r], mn, accm[i]);
            }
          }
        }
      }
    } else {  // Q6_K
      d = half_bits(*reinterpret_cast<const uint16_t*>(blk));
#pragma unroll QG_MFMA_UNROLL
      for (int grp = 0; grp < 8; ++grp) {
        // ql[8g .. 8g+7] and qh[0..7] of this 32-element group; the block is
        // only 2-byte aligned, so read 16-bit halves.
        const uint16_t* ql16 = reinterpret_cast<const uint16_t*>(blk + 18 + 16 * grp + 8 * g);
        const uint16_t* qh16 = reinterpret_cast<const uint16_t*>(blk + 146 + 8 * grp);
        const uint32_t ql0 = ql16[0] | ((uint32_t)ql16[1] << 16), ql1 = ql16[2] | ((uint32_t)ql16[3] << 16);
        const uint32_t qh0 = qh16[0] | ((uint32_t)qh16[1] << 16), qh1 = qh16[2] | ((uint32_t)qh16[3] << 16);
        const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(blk + 2 + 2 * grp);
        const uint32_t scs = sc16[0];
        const int sca = (int)(int8_t)(scs & 0xffu), scb = (int)(int8_t)(scs >> 8);
        // element 8g + c of sub-block a: low nibble of ql[8g + c], high bits
        // 2g..2g+1 of qh[c]; sub-block b: high nibble, bits 2(g + 2).
        const int sha = 2 * g, shb = 2 * g + 4;
        const uint32_t ca0 = minus32((ql0 & 0x0F0F0F0Fu) | (((qh0 >> sha) & 0x03030303u) << 4));
        const uint32_t ca1 = minus32((ql1 & 0x0F0F0F0Fu) | (((qh1 >> sha) & 0x03030303u) << 4));
        const uint32_t cb0 = minus32(((ql0 >> 4) & 0x0F0F0F0Fu) | (((qh0 >> shb) & 0x03030303u) << 4));
        const uint32_t cb1 = minus32(((ql1 >> 4) & 0x0F0F0F0Fu) | (((qh1 >> shb) & 0x03030303u) << 4));
        u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
        if (tok_ok) {
          a0 = *reinterpret_cast<const u32x4*>(xs + 32 * grp);
          a1 = *reinterpret_cast<const u32x4*>(xs + 32 * grp + 16);
        }
        const long aa = g ? pack2(a0.z, a0.w) : pack2(a0.x, a0.y);   // elements 8g .. 8g+7
        const long ab = g ? pack2(a1.z, a1.w) : pack2(a1.x, a1.y);   // elements 16 + 8g ..
        v16i Da = {0}, Db = {0};
        Da = __builtin_amdgcn_mfma_i32_32x32x16_i8(aa, pack2(ca0, ca1), Da, 0, 0, 0);
        Db = __builtin_amdgcn_mfma_i32_32x32x16_i8(ab, pack2(cb0, cb1), Db, 0, 0, 0);
        if constexpr (DOTS) {
          if (n < n_rows) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int tt = 8 * (i >> 2) + 4 * g + (i & 3);
              if (tt < m) {
                int32_t* o = dots + ((int64_t)tt * n_rows + n) * (k / 16) + (int64_t)sb * 16 + 2 * grp;
                o[0] = Da[i];
                o[1] = Db[i];
              }
            }
          }
        } else {
          const int bl = (sb - sb0) * 8 + grp;
          const float4* dxv = reinterpret_cast<const float4*>(sact + bl * kMT);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const float4 dd = dxv[2 * a4 + g];
            const float dl[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * a4 + r;
              accs[i] = fmaf(dl[r], (float)(Da[i] * sca + Db[i] * scb), accs[i]);
            }
          }
        }
      }
    }
    if constexpr (!DOTS) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = fmaf(d, accs[i], fmaf(-dmin, accm[i], acc[i]));
    }
  }

  if constexpr (!DOTS) {
    if (n < n_rows) {
      float* out = partials + (int64_t)split * kMT * n_rows;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tt = 8 * (i >> 2) + 4 * g + (i & 3);
        out[(int64_t)tt * n_rows + n] = acc[i];
      }
    }
  }
}

// y[t][n] = sum over splits, in split order.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ partials,
                                                           float* __restrict__ y, int64_t n_rows, int m,
                                                           int splits) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)m * n_rows) return;
  float s = 0.0f;
  for (int p = 0; p < splits; ++p) s += partials[(int64_t)p * kMT * n_rows + i];
  y[i] = s;
}

bool mfma_supported(int fmt) { return fmt == kQ4_K || fmt == kQ6_K; }

static void split_plan(int64_t k, int& splits, int& sb_per) {
  const int nsb = (int)(k / 256);
  // About 4 super-blocks per split: enough waves to cover the chip while
  // keeping the partial sums small.
  sb_per = nsb < 4 ? nsb : 4;
  splits = (nsb + sb_per - 1) / sb_per;
}

size_t gemm32_partials_bytes(int64_t n, int64_t k) {
  int splits, sb_per;
  split_plan(k, splits, sb_per);
  return (size_t)splits * kMT * n * sizeof(float);
}

template <int FMT, bool DOTS>
static hipError_t launch(const uint8_t* w, const int8_t* xq, const float* dx, const int32_t* sx,
                         float* partials, int32_t* dots, int64_t n, int64_t k, int m, hipStream_t s) {
  int splits, sb_per;
  split_plan(k, splits, sb_per);
  const int64_t tiles = (n + kRowsPerWave - 1) / kRowsPerWave;
  const unsigned gx = (unsigned)((tiles + kWaves - 1) / kWaves);
  const size_t lds = DOTS ? 16 : (size_t)2 * sb_per * 8 * kMT * sizeof(float);
  hipLaunchKernelGGL((gemm32_kernel<FMT, DOTS>), dim3(gx, (unsigned)splits), dim3(kWaves * 64), lds, s, w, xq,
                     dx, sx, partials, dots, n, k, m, splits, sb_per);
  return hipGetLastError();
}

hipError_t launch_gemm32(int fmt, const uint8_t* w, const int8_t* xq, const float* dx, const int32_t* sx,
                         float* y, float* partials, int64_t n, int64_t k, int m, hipStream_t s) {
  if (!mfma_supported(fmt) || m < 1 || m > kMT || k % 256) return hipErrorInvalidValue;
  hipError_t e = fmt == kQ4_K ? launch<kQ4_K, false>(w, xq, dx, sx, partials, nullptr, n, k, m, s)
                              : launch<kQ6_K, false>(w, xq, dx, sx, partials, nullptr, n, k, m, s);
  if (e != hipSuccess) return e;
  int splits, sb_per;
  split_plan(k, splits, sb_per);
  const int64_t total = (int64_t)m * n;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, partials, y, n,
                     m, splits);
  return hipGetLastError();
}

hipError_t launch_gemm32_dots(int fmt, const uint8_t* w, const int8_t* xq, int32_t* dots, int64_t n,
                              int64_t k, int m, hipStream_t s) {
  if (!mfma_supported(fmt) || m < 1 || m > kMT || k % 256) return hipErrorInvalidValue;
  return fmt == kQ4_K ? launch<kQ4_K, true>(w, xq, nullptr, nullptr, nullptr, dots, n, k, m, s)
                      : launch<kQ6_K, true>(w, xq, nullptr, nullptr, nullptr, dots, n, k, m, s);
}

}  // namespace qg
