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
// Memory: the operands of one MFMA come from 32 different rows (and 32
// tokens), so reading them straight from global memory touches 32 cache
// lines per load. Instead a workgroup (4 waves) owns a tile of 32 weight rows
// and walks K in chunks of 4 super-blocks: the chunk -- 32 row segments of 4
// contiguous super-blocks -- is read with coalesced 16-byte loads into LDS
// (the next chunk is already in flight in registers while the current one is
// computed) and each wave decodes one super-block of it from LDS. The
// activation codes come from a token-tiled copy ([block][token][32], written
// by the quantizer), where the 32 tokens of one block are 1 KB of contiguous
// memory. Each wave accumulates its super-blocks; the four waves' sums are
// added through LDS in wave order. When there are few row tiles, K is also
// split across workgroups and a second kernel adds the splits in order. No
// atomics: results are bitwise reproducible.
#include "common.cuh"
#include "internal.h"
#include "mfma.h"

#ifndef QG_MM_MINWG
#define QG_MM_MINWG 512   // with fewer than 256 row tiles, K is split to reach this many workgroups
#endif

namespace qg {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kMT = 32;                     // token tile
constexpr int kRows = 32;                   // weight rows per workgroup
constexpr int kNW = 4;                      // waves per workgroup = super-blocks per chunk
constexpr int kBufDword3 = 0x00020000;      // raw buffer resource, gfx9 family
constexpr int kNonTemporal = 2;             // weights are read once
constexpr uint32_t kNowhere = 0xF0000000u;  // offset past every resource: reads zeros

template <int FMT> struct Geo {
  static constexpr int BB = FMT == kQ4_K ? 144 : 210;    // bytes per super-block
  static constexpr int SEG = kNW * BB;                   // bytes of one row in a chunk
  static constexpr int NCH = (SEG + 15 + 15) / 16;       // 16-byte loads per row (any start alignment)
  static constexpr int PITCH = 16 * (NCH | 1);           // LDS row pitch: an odd number of 16-byte units
  static constexpr int LPT = (kRows * NCH + kNW * 64 - 1) / (kNW * 64);  // loads per thread
  static constexpr int TILE = kRows * PITCH;             // LDS bytes of one chunk
};

QG_DEV long pack2(uint32_t lo, uint32_t hi) { return (long)(((uint64_t)hi << 32) | lo); }

QG_DEV uint64_t ld64(__amdgpu_buffer_rsrc_t r, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return (uint64_t)v[0] | ((uint64_t)v[1] << 32);
}

// q - 32 for four 6-bit codes q in 0..63, one per byte, as signed int8:
// (q | 0x80) - 0x20 never borrows across bytes, and xor 0x80 recentres.
QG_DEV uint32_t minus32(uint32_t q) { return ((q | 0x80808080u) - 0x20202020u) ^ 0x80808080u; }

template <int FMT, bool DOTS>
__global__ __launch_bounds__(kNW * 64) void gemm32_kernel(const uint8_t* __restrict__ W,
                                                          const int8_t* __restrict__ xqt,
                                                          const float* __restrict__ dx,
                                                          const int32_t* __restrict__ sx,
                                                          float* __restrict__ out, int32_t* __restrict__ dots,
                                                          int64_t n_rows, int64_t k, int m, int sps) {
  using G = Geo<FMT>;
  constexpr int BB = G::BB;
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* wt = lds;                                      // one chunk of weights [row][PITCH]
  float* s_dx = reinterpret_cast<float*>(lds + G::TILE);  // [block][token] of this split
  const int64_t rb = (k / 256) * BB;
  const int nsb = (int)(k / 256);
  const int kblocks = (int)(k / 32);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, col = lane & 31;
  const int64_t row0 = (int64_t)blockIdx.x * kRows;
  const int64_t n = row0 + col;
  const int rows_here = (int)((n_rows - row0) < kRows ? (n_rows - row0) : kRows);
  const int split = blockIdx.y;
  const int sb_begin = split * sps;
  const int sb_end = (sb_begin + sps) < nsb ? (sb_begin + sps) : nsb;
  const int nkb = (sb_end - sb_begin) * 8;  // 32-element blocks of this split
  float* s_c = s_dx + nkb * kMT;

  if constexpr (!DOTS) {
    for (int i = threadIdx.x; i < nkb * kMT; i += kNW * 64) {
      const int b = i >> 5, t = i & 31;
      const int64_t gb = (int64_t)sb_begin * 8 + b;
      float d = 0.0f;
      if (t < m) d = dx[(int64_t)t * kblocks + gb];
      s_dx[i] = d;
      if constexpr (FMT == kQ4_K) s_c[i] = t < m ? d * (float)sx[(int64_t)t * kblocks + gb] : 0.0f;
    }
  }

  // Weights of the tile (rows past n_rows read zeros; the extent is rounded
  // up to 16 bytes, the readable padding after a matrix) and the token-tiled
  // activation codes (codes of tokens past m are never used: their rows of D
  // are dropped).
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(W + row0 * rb), 0, (int)((rows_here * rb + 15) & ~(int64_t)15), kBufDword3);
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(xqt), 0, kblocks * kMT * 32, kBufDword3);

  // Chunk c covers super-blocks sb_begin + 4c .. +3 of every row of the tile;
  // row r's bytes sit at wt + r * PITCH + (its start % 16).
  const int nchunks = (sb_end - sb_begin + kNW - 1) / kNW;
  u32x4 pre[G::LPT];
  auto issue = [&](int c) __attribute__((always_inline)) {
    const bool ok = c < nchunks;
    const int64_t sb0 = sb_begin + kNW * c;
#pragma unroll
    for (int i = 0; i < G::LPT; ++i) {
      const int p = threadIdx.x + kNW * 64 * i;
      const int r = p / G::NCH, ch = p - r * G::NCH;
      uint32_t off = kNowhere;
      if (ok && r < kRows) off = (uint32_t)(((int64_t)r * rb + sb0 * BB) & ~(int64_t)15) + 16u * ch;
      pre[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)off, 0, kNonTemporal);
    }
  };
  // This wave's activation codes for super-block sb, token col: Q4_K
  // elements 16 g .. 16 g + 15 of each sub-block; Q6_K elements 8 g .. 8 g + 7
  // (a) and 16 + 8 g .. (b) of each group.
  auto load_act = [&](int sb, u32x4 (&a)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t o = ((uint32_t)((sb * 8 + j) * kMT + col)) * 32u;
      if constexpr (FMT == kQ4_K) {
        a[j] = __builtin_amdgcn_raw_buffer_load_b128(ar, (int)(o + 16u * g), 0, 0);
      } else {
        const uint64_t va = ld64(ar, (int)(o + 8u * g));
        const uint64_t vb = ld64(ar, (int)(o + 16u + 8u * g));
        a[j] = u32x4{(uint32_t)va, (uint32_t)(va >> 32), (uint32_t)vb, (uint32_t)(vb >> 32)};
      }
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < G::LPT; ++i) {
      const int p = threadIdx.x + kNW * 64 * i;
      const int r = p / G::NCH, ch = p - r * G::NCH;
      if (r < kRows) *reinterpret_cast<u32x4*>(wt + r * G::PITCH + 16 * ch) = pre[i];
    }
  };

  float acc[16], accs[16], accm[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

  // One super-block from the LDS chunk; this lane's row's super-block starts
  // at LDS byte `base`.
  auto compute = [&](int sb, uint32_t base, const u32x4 (&a)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) { accs[i] = 0.0f; accm[i] = 0.0f; }
    const int bl0 = (sb - sb_begin) * 8;  // split-local block of the first sub-block
    float d = 0.0f, dmin = 0.0f;
    if constexpr (FMT == kQ4_K) {
      const u32x4 h = *reinterpret_cast<const u32x4*>(wt + base);
      d = half_bits(h.x & 0xffffu);
      dmin = half_bits(h.x >> 16);
      // 6-bit sc_j at bit 6 j, m_j at bit 48 + 6 j of the 96-bit stream.
      const uint64_t s_lo = (uint64_t)h.y | ((uint64_t)h.z << 32);
      const uint64_t s_hi = (uint64_t)h.z | ((uint64_t)h.w << 32);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(wt + base + 16 + 16 * j);
        const int sh = g ? 4 : 0;
        const long b0 = pack2((q.x >> sh) & 0x0F0F0F0Fu, (q.y >> sh) & 0x0F0F0F0Fu);
        const long b1 = pack2((q.z >> sh) & 0x0F0F0F0Fu, (q.w >> sh) & 0x0F0F0F0Fu);
        v16i D = {0};
        D = __builtin_amdgcn_mfma_i32_32x32x16_i8(pack2(a[j].x, a[j].y), b0, D, 0, 0, 0);
        D = __builtin_amdgcn_mfma_i32_32x32x16_i8(pack2(a[j].z, a[j].w), b1, D, 0, 0, 0);
        if constexpr (DOTS) {
          if (n < n_rows) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int tt = 8 * (i >> 2) + 4 * g + (i & 3);
              if (tt < m) dots[((int64_t)tt * n_rows + n) * kblocks + (int64_t)sb * 8 + j] = D[i];
            }
          }
        } else {
          const int sc = (int)((s_lo >> (6 * j)) & 63u);
          const float4* dxv = reinterpret_cast<const float4*>(s_dx + (bl0 + j) * kMT);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const float4 dd = dxv[2 * a4 + g];
            const float dl[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * a4 + r;
              accs[i] = fmaf(dl[r], (float)__mul24(D[i], sc), accs[i]);
            }
          }
        }
      }
      if constexpr (!DOTS) {
        // Min term sum_j c[t][j] m_j[n] of the super-block as a 32 x 8 by 8 x 32
        // fp32 product on the matrix cores (v_mfma_f32_32x32x2_f32, same D
        // layout): A[t][kk] = c of token col, block 2 s + kk (kk = g); B[kk][n]
        // = m_{2 s + kk} of this lane's row.
        v16f M = {0.0f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int jj = 2 * st + g;
          const float cval = s_c[(bl0 + jj) * kMT + col];
          const float mval = (float)((s_hi >> (16 + 6 * jj)) & 63u);
          M = __builtin_amdgcn_mfma_f32_32x32x2f32(cval, mval, M, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) accm[i] = M[i];
      }
    } else {
      d = half_bits(lds_u16(wt, base));
#pragma unroll
      for (int grp = 0; grp < 8; ++grp) {
        // Element 8g + c of sub-block a: low nibble of ql[16 grp + 8 g + c],
        // bits 2g..2g+1 of qh[8 grp + c]; sub-block b: high nibble, bits 2(g + 2).
        uint32_t ql[2], qh[2];
        lds_read_unaligned<2>(wt, base + 18 + 16 * grp + 8 * g, ql);
        lds_read_unaligned<2>(wt, base + 146 + 8 * grp, qh);
        const uint32_t scs = lds_u16(wt, base + 2 + 2 * grp);
        const int sha = 2 * g, shb = 2 * g + 4;
        const uint32_t ca0 = minus32((ql[0] & 0x0F0F0F0Fu) | (((qh[0] >> sha) & 0x03030303u) << 4));
        const uint32_t ca1 = minus32((ql[1] & 0x0F0F0F0Fu) | (((qh[1] >> sha) & 0x03030303u) << 4));
        const uint32_t cb0 = minus32(((ql[0] >> 4) & 0x0F0F0F0Fu) | (((qh[0] >> shb) & 0x03030303u) << 4));
        const uint32_t cb1 = minus32(((ql[1] >> 4) & 0x0F0F0F0Fu) | (((qh[1] >> shb) & 0x03030303u) << 4));
        v16i Da = {0}, Db = {0};
        Da = __builtin_amdgcn_mfma_i32_32x32x16_i8(pack2(a[grp].x, a[grp].y), pack2(ca0, ca1), Da, 0, 0, 0);
        Db = __builtin_amdgcn_mfma_i32_32x32x16_i8(pack2(a[grp].z, a[grp].w), pack2(cb0, cb1), Db, 0, 0, 0);
        if constexpr (DOTS) {
          if (n < n_rows) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int tt = 8 * (i >> 2) + 4 * g + (i & 3);
              if (tt < m) {
                int32_t* o2 = dots + ((int64_t)tt * n_rows + n) * (k / 16) + (int64_t)sb * 16 + 2 * grp;
                o2[0] = Da[i];
                o2[1] = Db[i];
              }
            }
          }
        } else {
          const int sca = (int)(int8_t)(scs & 0xffu), scb = (int)(int8_t)(scs >> 8);
          const float4* dxv = reinterpret_cast<const float4*>(s_dx + (bl0 + grp) * kMT);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const float4 dd = dxv[2 * a4 + g];
            const float dl[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * a4 + r;
              accs[i] = fmaf(dl[r], (float)(__mul24(Da[i], sca) + __mul24(Db[i], scb)), accs[i]);
            }
          }
        }
      }
    }
    if constexpr (!DOTS) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = fmaf(d, accs[i], fmaf(-dmin, accm[i], acc[i]));
    }
  };

  issue(0);
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();  // the previous chunk is no longer read (and dx is staged)
    store();
    __syncthreads();
    issue(c + 1);
    const int sb = sb_begin + kNW * c + wid;
    if (sb < sb_end) {
      u32x4 a[8];
      load_act(sb, a);
      const int64_t sb0 = sb_begin + kNW * c;
      const uint32_t base = (uint32_t)(col * G::PITCH) + (uint32_t)(((int64_t)col * rb + sb0 * BB) & 15) +
                            (uint32_t)(wid * BB);
      compute(sb, base, a);
    }
  }

  if constexpr (!DOTS) {
    // The waves' sums, added in wave order through LDS (the chunk area is free).
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);  // [kNW][16][64]
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(wid * 16 + i) * 64 + lane] = acc[i];
    __syncthreads();
    float* dst = out + (int64_t)split * kMT * n_rows;  // y itself when there is one split
    for (int o = threadIdx.x; o < 16 * 64; o += kNW * 64) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) s += red[w * 16 * 64 + o];
      const int i = o >> 6, l = o & 63;
      const int tt = 8 * (i >> 2) + 4 * (l >> 5) + (i & 3);
      const int64_t nn = row0 + (l & 31);
      if (tt < m && nn < n_rows) dst[(int64_t)tt * n_rows + nn] = s;
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

bool shape_ok(int fmt, int64_t n, int64_t k, int m) {
  // Buffer offsets are 32-bit: a tile's rows and the tiled activations must fit.
  const int64_t rb = (k / 256) * (fmt == kQ4_K ? 144 : 210);
  return (fmt == kQ4_K || fmt == kQ6_K) && m >= 1 && m <= kMT && k >= 256 && k % 256 == 0 && n >= 1 &&
         rb * kRows < (1ll << 30) && (k / 32) * kMT * 32 < (1ll << 30);
}

// Super-blocks per split: one split when the row tiles alone give every CU a
// workgroup, else K is shared out in whole chunks.
void split_plan(int64_t n, int64_t k, int& splits, int& sps) {
  const int64_t tiles = (n + kRows - 1) / kRows;
  const int nsb = (int)(k / 256);
  // Measured on MI355X: 384 row tiles run best unsplit; 128 tiles (4096
  // rows) best with K shared out four ways.
  int want = tiles >= 256 ? 1 : (int)((QG_MM_MINWG + tiles - 1) / tiles);
  const int maxs = nsb / kNW > 0 ? nsb / kNW : 1;
  if (want > maxs) want = maxs;
  sps = (nsb + want - 1) / want;
  sps = (sps + kNW - 1) / kNW * kNW;
  splits = (nsb + sps - 1) / sps;
}

template <int FMT, bool DOTS>
hipError_t launch_t(const uint8_t* w, const int8_t* xqt, const float* dx, const int32_t* sx, float* out,
                    int32_t* dots, int64_t n, int64_t k, int m, int splits, int sps, hipStream_t s) {
  using G = Geo<FMT>;
  auto kern = gemm32_kernel<FMT, DOTS>;
  const size_t stage = DOTS ? 0 : (size_t)sps * 8 * kMT * sizeof(float) * (FMT == kQ4_K ? 2 : 1);
  const size_t red = (size_t)kNW * 16 * 64 * sizeof(float);
  size_t lds = (size_t)G::TILE + stage;
  if (lds < red) lds = red;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  int per_cu = 0;  // raises the dynamic-LDS limit (once per kernel and device)
  hipError_t qe = kernel_residency(reinterpret_cast<const void*>(kern), kNW * 64, lds, true, &per_cu);
  if (qe != hipSuccess) return qe;
  const unsigned tiles = (unsigned)((n + kRows - 1) / kRows);
  hipLaunchKernelGGL(kern, dim3(tiles, (unsigned)splits), dim3(kNW * 64), lds, s, w, xqt, dx, sx, out, dots, n,
                     k, m, sps);
  return hipGetLastError();
}

}  // namespace

bool mfma_supported(int fmt) { return fmt == kQ4_K || fmt == kQ6_K; }

size_t gemm32_partials_bytes(int64_t n, int64_t k) {
  int splits, sps;
  split_plan(n, k, splits, sps);
  return splits > 1 ? (size_t)splits * kMT * n * sizeof(float) : 0;
}

size_t gemm32_tiled_act_bytes(int64_t k) { return (size_t)(k / 32) * kMT * 32; }

hipError_t launch_gemm32(int fmt, const uint8_t* w, const int8_t* xqt, const float* dx, const int32_t* sx,
                         float* y, float* partials, int64_t n, int64_t k, int m, hipStream_t s) {
  if (!shape_ok(fmt, n, k, m)) return hipErrorInvalidValue;
  int splits, sps;
  split_plan(n, k, splits, sps);
  if (splits > 1 && !partials) return hipErrorInvalidValue;
  float* out = splits > 1 ? partials : y;
  hipError_t e = fmt == kQ4_K ? launch_t<kQ4_K, false>(w, xqt, dx, sx, out, nullptr, n, k, m, splits, sps, s)
                              : launch_t<kQ6_K, false>(w, xqt, dx, sx, out, nullptr, n, k, m, splits, sps, s);
  if (e != hipSuccess || splits == 1) return e;
  const int64_t total = (int64_t)m * n;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, partials, y, n,
                     m, splits);
  return hipGetLastError();
}

hipError_t launch_gemm32_dots(int fmt, const uint8_t* w, const int8_t* xqt, int32_t* dots, int64_t n,
                              int64_t k, int m, hipStream_t s) {
  if (!shape_ok(fmt, n, k, m)) return hipErrorInvalidValue;
  int splits, sps;
  split_plan(n, k, splits, sps);
  return fmt == kQ4_K
             ? launch_t<kQ4_K, true>(w, xqt, nullptr, nullptr, nullptr, dots, n, k, m, splits, sps, s)
             : launch_t<kQ6_K, true>(w, xqt, nullptr, nullptr, nullptr, dots, n, k, m, splits, sps, s);
}

}  // namespace qg
