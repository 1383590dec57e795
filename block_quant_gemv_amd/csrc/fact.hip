// Float-activation batched GEMV for the 32-element block formats (Q4_0,
// Q8_0): y[m, n] = x[m, k] . W_hat[n, k]^T with the activations kept in
// fp32, no activation quantization. In prefill, int8 activations cost about
// 3 % perplexity where float activations cost about 0.2 % ("01 · Phase
// overview: from 2B to 8B to MoE", icman.com.cn, issue ledger item ⑮), so
// this is the batched path's accuracy variant.
//
// The product is a dense contraction over up to 32 tokens, so it runs on
// fp32 matrix cores: v_mfma_f32_16x16x4_f32 takes a 16 x 4 tile of weights
// (lane = row + 16 g) and a 4 x 16 tile of activations (lane = token + 16 g)
// and accumulates the 16 x 16 products in fp32. Each weight value d * q is
// exact in fp32 (an 11-bit fp16 significand times a code of at most 8 bits).
// Within one 32-element block, lane group g owns elements 8 g .. 8 g + 7 for
// both operands, so step s of 8 feeds element 8 g + s of the weights and of
// the activations; the k-order inside an MFMA does not change the sum.
//
// A workgroup computes 16 rows for all tokens; its 4 waves take the row
// tile's blocks in turn (wave w: blocks w, w + 4, ...), so at any time the 4
// waves read neighbouring blocks of the same 16 rows; each wave loads several
// of its blocks before it multiplies them. The 4 partial tiles are
// added in wave order through LDS, and wave 0 stores y.
#include "common.cuh"
#include "fact.h"
#include "internal.h"

namespace qg {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef QG_FA_ROWS
#define QG_FA_ROWS 1  // one to four tokens take the row-streaming kernel
#endif
#ifndef QG_FA_WAVES
#define QG_FA_WAVES 4
#endif
constexpr int kFaWaves = QG_FA_WAVES;  // waves per workgroup, splitting the row tile's blocks
#ifndef QG_FA_UNROLL
#define QG_FA_UNROLL 1  // measured: 4 and 8 are slower (the loads are not latency-bound)
#endif
constexpr int kFaUnroll = QG_FA_UNROLL;  // blocks per wave per loop iteration

// Bytes per block: fp16 d, then the codes (Q4_0: 16 bytes of nibbles, element
// e < 16 in the low nibble of byte e, element e >= 16 in the high nibble of
// byte e - 16; Q8_0: 32 int8 codes).
template <int FMT>
constexpr int kFaBlockBytes = FMT == 1 ? 18 : 34;

// The 8 dequantized weights of elements 8 g .. 8 g + 7 of one block (2-byte
// aligned loads: blocks are 18 or 34 bytes long).
template <int FMT>
QG_DEV void fa_weights(const uint8_t* __restrict__ blk, int g, float (&w)[8]) {
  const uint16_t* p16 = reinterpret_cast<const uint16_t*>(blk);
  const float d = half_bits(p16[0]);
  if constexpr (FMT == 2) {
    const uint16_t* c = p16 + 1 + 4 * g;  // bytes 2 + 8 g ..
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = c[i];
      w[2 * i] = d * (float)(int8_t)(v & 0xffu);
      w[2 * i + 1] = d * (float)(int8_t)(v >> 8);
    }
  } else {
    const uint16_t* c = p16 + 1 + 4 * (g & 1);  // bytes 2 + 8 (g & 1) ..
    const int sh = g < 2 ? 0 : 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = c[i];
      w[2 * i] = d * (float)((int)((v >> sh) & 0xfu) - 8);
      w[2 * i + 1] = d * (float)((int)((v >> (8 + sh)) & 0xfu) - 8);
    }
  }
}

QG_DEV void fa_acts(const float* __restrict__ p, float (&a)[8]) {
  const float4 u = reinterpret_cast<const float4*>(p)[0];
  const float4 v = reinterpret_cast<const float4*>(p)[1];
  a[0] = u.x, a[1] = u.y, a[2] = u.z, a[3] = u.w, a[4] = v.x, a[5] = v.y, a[6] = v.z, a[7] = v.w;
}

// NT: token tiles of 16 (1 for m <= 16, 2 for m <= 32).
template <int FMT, int NT>
__global__ __launch_bounds__(kFaWaves * 64) void fact_kernel(const uint8_t* __restrict__ w,
                                                             const float* __restrict__ x, float* __restrict__ y,
                                                             int m, int64_t n, int64_t k) {
  constexpr int BB = kFaBlockBytes<FMT>;
  __shared__ f32x4 red[kFaWaves][NT][64];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15;  // weight row of the A operand, token of the B operand
  const int g = lane >> 4;  // element group within a block
  const int64_t r0 = (int64_t)blockIdx.x * 16;
  const int64_t nb = k / 32;
  const bool row_ok = r0 + i < n;
  const uint8_t* wr = w + (row_ok ? r0 + i : 0) * nb * BB;
  bool tok_ok[NT];
  const float* xr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    tok_ok[t] = 16 * t + i < m;
    xr[t] = x + (int64_t)(tok_ok[t] ? 16 * t + i : 0) * k + 8 * g;
  }
  // Two accumulators per token tile (even and odd steps) so consecutive
  // MFMAs do not wait on each other's result.
  f32x4 acc[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t][0] = acc[t][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // kFaUnroll blocks per iteration: all their loads are issued before the
  // first MFMA, so one memory latency covers several blocks. A block past
  // the end contributes zeros.
  for (int64_t b0 = wid; b0 < nb; b0 += kFaWaves * kFaUnroll) {
    float wv[kFaUnroll][8];
    float xa[kFaUnroll][NT][8];
#pragma unroll
    for (int u = 0; u < kFaUnroll; ++u) {
      // Loads are unconditional, from clamped (always valid) addresses, and
      // the values of a row, token or block out of range are then replaced
      // by zeros: no load sits in a divergent branch whose other side would
      // have to wait for it.
      const int64_t b = b0 + (int64_t)u * kFaWaves;
      const bool ok = b < nb;
      const int64_t bc = ok ? b : nb - 1;
      fa_weights<FMT>(wr + bc * BB, g, wv[u]);
      const bool wok = row_ok && ok;
#pragma unroll
      for (int s = 0; s < 8; ++s) wv[u][s] = wok ? wv[u][s] : 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        fa_acts(xr[t] + bc * 32, xa[u][t]);
        const bool xok = tok_ok[t] && ok;
#pragma unroll
        for (int s = 0; s < 8; ++s) xa[u][t][s] = xok ? xa[u][t][s] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kFaUnroll; ++u) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t][s & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[u][s], xa[u][t][s], acc[t][s & 1], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) red[wid][t][lane] = acc[t][0] + acc[t][1];
  __syncthreads();
  if (wid != 0) return;
  // Output lane layout: token 16 t + (lane & 15), rows r0 + 4 g + 0..3.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4 v = red[0][t][lane];
#pragma unroll
    for (int ww = 1; ww < kFaWaves; ++ww) v += red[ww][t][lane];
    const int tok = 16 * t + i;
    if (tok >= m) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = r0 + 4 * g + r;
      if (row < n) y[(int64_t)tok * n + row] = v[r];
    }
  }
}

// One to four tokens: the matrix cores would do up to 16 times the useful
// work, and per-lane 2-byte code loads do not coalesce, so the rows stream
// like the decode GEMV's: a wave copies one row at a time into its own LDS
// tile with 16-byte loads that are contiguous across lanes (the next row is
// requested as soon as the current one is in LDS), and each lane takes 32-
// element blocks b = lane, lane + 64, ...: an fp32 dot of its codes (read
// from the tile at any 2-byte alignment) with x, staged once per workgroup in
// LDS, then times the block scale. The 64 lanes of a row are summed in a
// fixed order, so results are bitwise reproducible.
constexpr int kRowWaves = 4;
constexpr int kRowLpl = 5;                       // 16-byte loads per lane per row
constexpr int kRowTile = kRowLpl * 64 * 16;      // LDS bytes of a wave's row tile
constexpr int64_t kRowMaxBytes = kRowTile - 30;  // the row plus its alignment chunks must fit

template <int FMT, int MT>
__global__ __launch_bounds__(kRowWaves * 64) void fact_rows_kernel(const uint8_t* __restrict__ w,
                                                                   const float* __restrict__ x,
                                                                   float* __restrict__ y, int m, int64_t n,
                                                                   int64_t k) {
  constexpr int BB = kFaBlockBytes<FMT>;
  extern __shared__ __align__(16) uint8_t smem[];
  // x of token t in LDS by quarter blocks: float4 v (elements 4v .. 4v + 3)
  // of block b at slot t * k / 4 + v * nb + b, so that the 64 lanes of a
  // wave, reading quarter v of blocks lane, lane + 64, ..., read consecutive
  // 16-byte words (the plain layout puts them 128 bytes apart: bank
  // conflicts).
  float* xs = reinterpret_cast<float*>(smem);
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* tile = smem + (size_t)MT * k * 4 + (size_t)wid * kRowTile;
  const int64_t nb = k / 32;
  const int64_t rb = nb * BB;
  const int64_t gw = (int64_t)blockIdx.x * kRowWaves + wid;
  const int64_t nw = (int64_t)gridDim.x * kRowWaves;

  // The 16-byte chunks spanning row r, through a buffer resource that covers
  // exactly them (rows past the end: no chunks, the loads read zeros).
  auto chunks = [&](int64_t r, int64_t& a0) __attribute__((always_inline)) -> int {
    if (r >= n) { a0 = 0; return 0; }
    a0 = (r * rb) & ~(int64_t)15;
    return (int)((((r * rb + rb + 15) & ~(int64_t)15) - a0) >> 4);
  };
  u32x4 buf[kRowLpl];
  auto issue = [&](int64_t r) __attribute__((always_inline)) {
    int64_t a0;
    const int nch = chunks(r, a0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w + a0), 0, nch * 16, 0x00020000);
#pragma unroll
    for (int i = 0; i < kRowLpl; ++i) buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + 64 * i) * 16, 0, 2);
  };
  issue(gw);

  // x of every token into LDS (tokens past m read as zeros), in batches of
  // four 16-byte loads per thread, all issued before any is stored: one
  // memory round trip per batch.
  const int64_t nx = (int64_t)MT * k / 4;
  for (int64_t i0 = threadIdx.x; i0 < nx; i0 += 4 * kRowWaves * 64) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * kRowWaves * 64;
      v[u] = (i < nx && (4 * i) / k < m) ? reinterpret_cast<const float4*>(x)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * kRowWaves * 64;
      if (i < nx) {
        const int64_t t = (4 * i) / k, j = i - t * (k / 4);  // token, float4 within the token
        reinterpret_cast<float4*>(xs)[t * (k / 4) + (j & 7) * nb + (j >> 3)] = v[u];
      }
    }
  }
  __syncthreads();

  for (int64_t r = gw; r < n; r += nw) {
    int64_t a0;
    const int nch = chunks(r, a0);
    __builtin_amdgcn_wave_barrier();  // the previous row's tile reads are done
#pragma unroll
    for (int i = 0; i < kRowLpl; ++i)
      if (lane + 64 * i < nch) *reinterpret_cast<u32x4*>(tile + 16 * (lane + 64 * i)) = buf[i];
    issue(r + nw);
    __builtin_amdgcn_wave_barrier();  // the tile is written before any lane reads it
    const uint32_t base = (uint32_t)(r * rb - a0);
    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
    for (int64_t b = lane; b < nb; b += 64) {
      const uint32_t o = base + (uint32_t)(b * BB);
      const float d = half_bits(lds_u16(tile, o));
      float q[32];
      if constexpr (FMT == 2) {
        uint32_t c[8];
        lds_read4_direct(tile, o + 2, *reinterpret_cast<uint32_t(*)[4]>(c));
        lds_read4_direct(tile, o + 18, *reinterpret_cast<uint32_t(*)[4]>(c + 4));
#pragma unroll
        for (int i = 0; i < 32; ++i) q[i] = (float)(int8_t)(c[i / 4] >> (8 * (i % 4)));
      } else {
        uint32_t c[4];
        lds_read4_direct(tile, o + 2, c);
        // element e < 16: low nibble of byte e; e >= 16: high nibble of byte e - 16
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          q[i] = (float)((int)((c[i / 4] >> (8 * (i % 4))) & 0xfu) - 8);
          q[16 + i] = (float)((int)((c[i / 4] >> (8 * (i % 4) + 4)) & 0xfu) - 8);
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float4* xv = reinterpret_cast<const float4*>(xs) + (int64_t)t * (k / 4) + b;
        float sdot = 0.0f;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float4 f = xv[v * nb];
          sdot = fmaf(q[4 * v], f.x, sdot);
          sdot = fmaf(q[4 * v + 1], f.y, sdot);
          sdot = fmaf(q[4 * v + 2], f.z, sdot);
          sdot = fmaf(q[4 * v + 3], f.w, sdot);
        }
        acc[t] = fmaf(d, sdot, acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float v = group_sum(acc[t], 64);
      if (lane == 0 && t < m) y[(int64_t)t * n + r] = v;
    }
  }
}

template <int FMT, int MT>
hipError_t launch_rows_t(const uint8_t* w, const float* x, float* y, int m, int64_t n, int64_t k, hipStream_t s) {
  auto kern = fact_rows_kernel<FMT, MT>;
  const size_t lds = (size_t)MT * k * 4 + (size_t)kRowWaves * kRowTile;
  int per_cu = 0, cus = 0;
  hipError_t qe = kernel_residency(reinterpret_cast<const void*>(kern), kRowWaves * 64, lds, true, &per_cu, &cus);
  if (qe != hipSuccess) return qe;
  if (per_cu < 1) return hipErrorInvalidValue;
  int64_t wgs = (int64_t)cus * per_cu;
  const int64_t need = (n + kRowWaves - 1) / kRowWaves;
  if (wgs > need) wgs = need;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kRowWaves * 64), lds, s, w, x, y, m, n, k);
  return hipGetLastError();
}

// The row-streaming kernel's shapes: up to four tokens whose x fits 64 KB of
// LDS next to the row tiles, and rows of at most kRowMaxBytes.
bool rows_ok(int fmt, int m, int64_t k) {
  const int64_t rb = k / 32 * (fmt == 1 ? 18 : 34);
  const int mt = m <= 1 ? 1 : m <= 2 ? 2 : 4;
  return QG_FA_ROWS && m <= 4 && rb <= kRowMaxBytes && (int64_t)mt * k * 4 + kRowWaves * kRowTile <= 64 * 1024;
}

template <int FMT>
hipError_t launch_rows(const uint8_t* w, const float* x, float* y, int m, int64_t n, int64_t k, hipStream_t s) {
  if (m <= 1) return launch_rows_t<FMT, 1>(w, x, y, m, n, k, s);
  if (m <= 2) return launch_rows_t<FMT, 2>(w, x, y, m, n, k, s);
  return launch_rows_t<FMT, 4>(w, x, y, m, n, k, s);
}

}  // namespace

bool fact_supported(int fmt) { return fmt == 1 || fmt == 2; }

hipError_t launch_fact(int fmt, const uint8_t* w, const float* x, float* y, int m, int64_t n, int64_t k,
                       hipStream_t s) {
  if (!fact_supported(fmt) || m < 1 || m > 32 || n < 1 || k < 32 || k % 32) return hipErrorInvalidValue;
  if (rows_ok(fmt, m, k)) return fmt == 1 ? launch_rows<1>(w, x, y, m, n, k, s) : launch_rows<2>(w, x, y, m, n, k, s);
  const dim3 grid((unsigned)((n + 15) / 16)), block(kFaWaves * 64);
  if (fmt == 1) {
    if (m <= 16) hipLaunchKernelGGL((fact_kernel<1, 1>), grid, block, 0, s, w, x, y, m, n, k);
    else hipLaunchKernelGGL((fact_kernel<1, 2>), grid, block, 0, s, w, x, y, m, n, k);
  } else {
    if (m <= 16) hipLaunchKernelGGL((fact_kernel<2, 1>), grid, block, 0, s, w, x, y, m, n, k);
    else hipLaunchKernelGGL((fact_kernel<2, 2>), grid, block, 0, s, w, x, y, m, n, k);
  }
  return hipGetLastError();
}

}  // namespace qg
