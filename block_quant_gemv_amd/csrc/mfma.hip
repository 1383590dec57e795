// Batched (9..32 tokens per launch tile) GEMM over packed Q4_K / Q6_K
// weights with int8 MFMA, gfx950.
//
// With 32 tokens the work is a real dense contraction: the vector int8 dot
// products of the decode GEMV would make the VALU the bottleneck, so the
// integer block dots run on the matrix cores instead (the prefill/batched
// case of "01 · Phase overview: from 2B to 8B to MoE", icman.com.cn, section
// 九: at batch 32 the dp4a path was exhausted and matrix cores were needed).
// Every MFMA stays inside one scale group -- a 32-element Q4_K sub-block, or
// a 16-element Q6_K sub-block with the other half of the weight operand
// zeroed -- because each group has its own scale (and min), applied in fp32
// after the integer product.
//
// v_mfma_i32_16x16x32_i8, D[m][n] += sum_k A[m][k] B[k][n], lane l, g = l / 16:
//   A (16 x 32): A[l % 16][8 g .. 8 g + 7]        (m = token)
//   B (32 x 16): B[8 g .. 8 g + 7][l % 16]        (n = weight row)
//   D (16 x 16): D[4 g + i][l % 16], i < 4
// so each lane owns one weight row (its scale fields are per-lane values)
// and four tokens of each 16-token half. Q4_K's min term, sum_j (dx s)[t][j]
// m_j[n], is a real contraction over sub-blocks: two fp32 matrix-core
// products (v_mfma_f32_16x16x4f32) per super-block and token half, added
// straight into the accumulators.
//
// Work: a workgroup owns 16 weight rows for all 32 tokens and splits K over
// its waves; each wave streams its own super-blocks (16 row segments read
// with coalesced 16-byte loads, two super-blocks in flight in registers)
// through a wave-private LDS tile from which each lane reads its row's
// fields, and keeps its partial sums in registers. The waves' sums are added
// through LDS in wave order at the end, so results are bitwise reproducible
// with no atomics and no second launch. 16-row tiles give 768 workgroups for
// 12288 rows, three per CU on 256 CUs (of 8 waves each: two super-blocks per
// wave at K = 4096); 4096 rows at K = 12288 run 256 workgroups of 16 waves.
#include "common.cuh"
#include "internal.h"
#include "mfma.h"

namespace qg {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMT = 32;                     // token tile
constexpr int kRows = 16;                   // weight rows per workgroup
constexpr int kBufDword3 = 0x00020000;      // raw buffer resource, gfx9 family
constexpr int kNonTemporal = 2;             // weights are read once
constexpr uint32_t kNowhere = 0xF0000000u;  // offset past every resource: reads zeros

template <int FMT> struct Geo {
  static constexpr int BB = FMT == kQ4_K ? 144 : 210;        // bytes per super-block
  static constexpr int NCH = FMT == kQ4_K ? 9 : 15;          // 16-byte chunks per row segment (any alignment)
  static constexpr int PITCH = 16 * NCH;                     // LDS row pitch: an odd number of 16-byte units
  static constexpr int LPL = (kRows * NCH + 63) / 64;        // loads per lane per super-block
  static constexpr int TILE = kRows * PITCH;                 // LDS bytes of one wave's tile
};

QG_DEV long pack2(uint32_t lo, uint32_t hi) { return (long)(((uint64_t)hi << 32) | lo); }

// q - 32 for four 6-bit codes q in 0..63, one per byte, as signed int8:
// (q | 0x80) - 0x20 never borrows across bytes, and xor 0x80 recentres.
QG_DEV uint32_t minus32(uint32_t q) { return ((q | 0x80808080u) - 0x20202020u) ^ 0x80808080u; }

// Per-wave shared memory: the super-block tile and the staged per-block
// activation scales of the wave's K range ([block][token]).
template <int FMT>
struct WaveLds {
  __host__ __device__ static size_t bytes(int spw) {
    return (size_t)Geo<FMT>::TILE + (size_t)spw * 8 * kMT * 4;
  }
};

template <int FMT, int NW, bool DOTS>
__global__ __launch_bounds__(NW * 64, 3) void gemm32_kernel(const uint8_t* __restrict__ W,
                                                         const int8_t* __restrict__ xqt,
                                                         const float* __restrict__ dxt,
                                                         const float* __restrict__ cxt,
                                                         float* __restrict__ y, int32_t* __restrict__ dots,
                                                         int64_t n_rows, int64_t k, int m, int spw) {
  using G = Geo<FMT>;
  constexpr int BB = G::BB;
  extern __shared__ __align__(16) uint8_t lds[];
  const int64_t rb = (k / 256) * BB;
  const int nsb = (int)(k / 256);
  const int kblocks = (int)(k / 32);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.x * kRows;
  const int64_t n = row0 + col;
  const int rows_here = (int)((n_rows - row0) < kRows ? (n_rows - row0) : kRows);
  const int sb_begin = wid * spw;
  const int sb_end = (sb_begin + spw) < nsb ? (sb_begin + spw) : nsb;
  const int nmine = sb_end > sb_begin ? sb_end - sb_begin : 0;
  const size_t wave_bytes = WaveLds<FMT>::bytes(spw);
  uint8_t* tile = lds + (size_t)wid * wave_bytes;
  float* s_dx = reinterpret_cast<float*>(tile + G::TILE);   // [local block][token]

  // Weights of the tile: rows past n_rows read zeros (the extent is rounded
  // up to 16 bytes, the readable padding after a matrix).
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(W + row0 * rb), 0, (int)((rows_here * rb + 15) & ~(int64_t)15), kBufDword3);
  // Block-major activation codes (1 KB per block); token slots past m hold
  // anything (their rows of D are dropped).
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(xqt), 0, kblocks * kMT * 32, kBufDword3);

  // Chunk c of a super-block's 16 row segments: row c / NCH, 16-byte chunk
  // c % NCH of the row's aligned span; row r lands at tile + r * PITCH.
  auto issue = [&](u32x4 (&buf)[G::LPL], int sb) __attribute__((always_inline)) {
    const bool ok = sb < sb_end;
#pragma unroll
    for (int i = 0; i < G::LPL; ++i) {
      const int c = lane + 64 * i;
      const int r = c / G::NCH, ch = c - r * G::NCH;
      uint32_t off = kNowhere;
      if (ok && r < kRows) off = (uint32_t)(((int64_t)r * rb + (int64_t)sb * BB) & ~(int64_t)15) + 16u * ch;
      buf[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)off, 0, kNonTemporal);
    }
  };
  auto store = [&](const u32x4 (&buf)[G::LPL]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < G::LPL; ++i) {
      const int c = lane + 64 * i;
      const int r = c / G::NCH, ch = c - r * G::NCH;
      if (r < kRows) *reinterpret_cast<u32x4*>(tile + r * G::PITCH + 16 * ch) = buf[i];
    }
  };
  // This lane's activation operands for the 32-element group (global block)
  // b: tokens col (half 0) and 16 + col (half 1), elements 8 g .. 8 g + 7,
  // which the block-major layout keeps in one 16-byte piece.
  auto load_act = [&](int64_t b, long& a0, long& a1) __attribute__((always_inline)) {
    const uint32_t o = (uint32_t)(b * 1024) + 16u * (uint32_t)lane;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ar, (int)o, 0, 0);
    a0 = pack2(v[0], v[1]);
    a1 = pack2(v[2], v[3]);
  };

  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};  // tokens 4g + i, 16 + 4g + i

  // The wave's per-block activation scales, contiguous in the block-major
  // layout, in batches of four 16-byte loads per lane; token
  // slots past m become zero. The first batch (the whole range when a wave
  // has at most four super-blocks) is requested before the weights: loads
  // return in issue order, so storing it waits for no weights.
  const int nvec = DOTS ? 0 : nmine * 8 * kMT / 4;  // float4s of the wave's range
  const float4* gdx = reinterpret_cast<const float4*>(dxt + (int64_t)sb_begin * 8 * kMT);
  float4 vd[4];
  auto load_scales = [&](int v0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = v0 + lane + 64 * i;
      if (v < nvec) {
        vd[i] = gdx[v];
      }
    }
  };
  auto store_scales = [&](int v0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = v0 + lane + 64 * i;
      if (v < nvec) {
        const int t = (4 * v) & (kMT - 1);  // token of the first of the four
        float4 d = vd[i];
        d.x = t + 0 < m ? d.x : 0.0f;
        d.y = t + 1 < m ? d.y : 0.0f;
        d.z = t + 2 < m ? d.z : 0.0f;
        d.w = t + 3 < m ? d.w : 0.0f;
        reinterpret_cast<float4*>(s_dx)[v] = d;
      }
    }
  };
  if constexpr (!DOTS) load_scales(0);

  // Weights two super-blocks ahead in registers (double buffer); the
  // activation operands of a super-block are requested when its step starts,
  // and the weights two ahead at its end, and other waves on the SIMD cover
  // the L2 latency of the activations.
  u32x4 bufA[G::LPL], bufB[G::LPL];
  issue(bufA, sb_begin);
  issue(bufB, sb_begin + 1);

  if constexpr (!DOTS) {
    store_scales(0);
    for (int v0 = 4 * 64; v0 < nvec; v0 += 4 * 64) {
      load_scales(v0);
      store_scales(v0);
    }
  }
  // One super-block: its weights from the registers to the wave's LDS tile,
  // its activations requested, the products from the tile, then the weights
  // two ahead requested into the freed registers.
  auto step = [&](int sb, u32x4 (&buf)[G::LPL]) __attribute__((always_inline)) {
    const int bl0 = (sb - sb_begin) * 8;         // wave-local block of the first group
    __builtin_amdgcn_wave_barrier();  // the previous super-block's tile reads are done
    store(buf);
    long act[8][2];
#pragma unroll
    for (int j = 0; j < 8; ++j) load_act((int64_t)sb * 8 + j, act[j][0], act[j][1]);
    // Q4_K's min-term operands: (dx s)[token][sub-block 4 q + g] for the
    // lane's token of each half (the block-major scale copy, from L2).
    float cm[2][2];
    if constexpr (FMT == kQ4_K && !DOTS) {
#pragma unroll
      for (int qd = 0; qd < 2; ++qd) {
        const float* c = cxt + ((int64_t)sb * 8 + 4 * qd + g) * kMT;
        cm[qd][0] = col < m ? c[col] : 0.0f;
        cm[qd][1] = 16 + col < m ? c[16 + col] : 0.0f;
      }
    }
    __builtin_amdgcn_wave_barrier();  // the tile is written before any lane reads it
    const uint32_t base = (uint32_t)(col * G::PITCH) + (uint32_t)(((int64_t)col * rb + (int64_t)sb * BB) & 15);
    v4f accs0 = {0.f, 0.f, 0.f, 0.f}, accs1 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == kQ4_K) {
      const u32x4 h = *reinterpret_cast<const u32x4*>(tile + base);
      const float d = half_bits(h.x & 0xffffu);
      const float dmin = half_bits(h.x >> 16);
      // 6-bit sc_j at bit 6 j, m_j at bit 48 + 6 j of the 96-bit stream.
      const uint64_t s_lo = (uint64_t)h.y | ((uint64_t)h.z << 32);
      const uint64_t s_hi = (uint64_t)h.z | ((uint64_t)h.w << 32);
      const int sh = (g >> 1) * 4;  // lane groups 2, 3 take the high nibbles (elements 16..31)
      if constexpr (!DOTS) {
        // Min term on fp32 matrix cores, straight into the accumulators: for
        // sub-blocks 4 q .. 4 q + 3, D[t][n] += sum_k (dx s)[t][4 q + k] *
        // (-dmin m_{4 q + k})[n] (v_mfma_f32_16x16x4f32: A[t][k] in lane
        // t + 16 k, B[k][n] in lane n + 16 k, D as for the integer products).
#pragma unroll
        for (int qd = 0; qd < 2; ++qd) {
          const int jj = 4 * qd + g;
          const float bm = -dmin * (float)((uint32_t)(s_hi >> (16 + 6 * jj)) & 63u);
          const float a0 = cm[qd][0], a1 = cm[qd][1];
          acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bm, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bm, acc1, 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint2 q = *reinterpret_cast<const uint2*>(tile + base + 16 + 16 * j + 8 * (g & 1));
        const long b = pack2((q.x >> sh) & 0x0F0F0F0Fu, (q.y >> sh) & 0x0F0F0F0Fu);
        v4i D0 = {0, 0, 0, 0}, D1 = {0, 0, 0, 0};
        D0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(act[j][0], b, D0, 0, 0, 0);
        D1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(act[j][1], b, D1, 0, 0, 0);
        if constexpr (DOTS) {
          if (n < n_rows) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t0 = 4 * g + i, t1 = 16 + 4 * g + i;
              if (t0 < m) dots[((int64_t)t0 * n_rows + n) * kblocks + (int64_t)sb * 8 + j] = D0[i];
              if (t1 < m) dots[((int64_t)t1 * n_rows + n) * kblocks + (int64_t)sb * 8 + j] = D1[i];
            }
          }
        } else {
          const int sc = (int)((s_lo >> (6 * j)) & 63u);
          const float4 d0 = *reinterpret_cast<const float4*>(s_dx + (bl0 + j) * kMT + 4 * g);
          const float4 d1 = *reinterpret_cast<const float4*>(s_dx + (bl0 + j) * kMT + 16 + 4 * g);
          accs0[0] = fmaf(d0.x, (float)__mul24(D0[0], sc), accs0[0]);
          accs0[1] = fmaf(d0.y, (float)__mul24(D0[1], sc), accs0[1]);
          accs0[2] = fmaf(d0.z, (float)__mul24(D0[2], sc), accs0[2]);
          accs0[3] = fmaf(d0.w, (float)__mul24(D0[3], sc), accs0[3]);
          accs1[0] = fmaf(d1.x, (float)__mul24(D1[0], sc), accs1[0]);
          accs1[1] = fmaf(d1.y, (float)__mul24(D1[1], sc), accs1[1]);
          accs1[2] = fmaf(d1.z, (float)__mul24(D1[2], sc), accs1[2]);
          accs1[3] = fmaf(d1.w, (float)__mul24(D1[3], sc), accs1[3]);
        }
      }
      if constexpr (!DOTS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc0[i] = fmaf(d, accs0[i], acc0[i]);
          acc1[i] = fmaf(d, accs1[i], acc1[i]);
        }
      }
    } else {
      const float d = half_bits(lds_u16(tile, base));
#pragma unroll
      for (int grp = 0; grp < 8; ++grp) {
        // Elements 8 (g & 1) .. + 7 of 16-element sub-block (g >> 1): low
        // 4 bits in ql[16 grp + 8 (g & 1) + c] (low nibble for sub-block a,
        // high for b), high 2 bits at bits 2 (g & 1) + 4 (g >> 1) of
        // qh[8 grp + c].
        uint32_t ql[2], qh[2];
        lds_read_unaligned<2>(tile, base + 18 + 16 * grp + 8 * (g & 1), ql);
        lds_read_unaligned<2>(tile, base + 146 + 8 * grp, qh);
        const uint32_t scs = lds_u16(tile, base + 2 + 2 * grp);
        const int lsh = 4 * (g >> 1), hsh = 2 * (g & 1) + 4 * (g >> 1);
        const uint32_t c0 = minus32(((ql[0] >> lsh) & 0x0F0F0F0Fu) | (((qh[0] >> hsh) & 0x03030303u) << 4));
        const uint32_t c1 = minus32(((ql[1] >> lsh) & 0x0F0F0F0Fu) | (((qh[1] >> hsh) & 0x03030303u) << 4));
        // Lane group g holds elements 8g..8g+7 of the 32-element group: groups
        // 0, 1 are sub-block a, groups 2, 3 sub-block b. One product per
        // sub-block, with the other sub-block's operand lanes zeroed.
        const long ba = (g < 2) ? pack2(c0, c1) : 0l;
        const long bb = (g >= 2) ? pack2(c0, c1) : 0l;
        v4i Pa0 = {0, 0, 0, 0}, Pa1 = {0, 0, 0, 0}, Pb0 = {0, 0, 0, 0}, Pb1 = {0, 0, 0, 0};
        Pa0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(act[grp][0], ba, Pa0, 0, 0, 0);
        Pa1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(act[grp][1], ba, Pa1, 0, 0, 0);
        Pb0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(act[grp][0], bb, Pb0, 0, 0, 0);
        Pb1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(act[grp][1], bb, Pb1, 0, 0, 0);
        if constexpr (DOTS) {
          if (n < n_rows) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t0 = 4 * g + i, t1 = 16 + 4 * g + i;
              const int64_t jo = (int64_t)sb * 16 + 2 * grp;
              if (t0 < m) {
                int32_t* o = dots + ((int64_t)t0 * n_rows + n) * (k / 16) + jo;
                o[0] = Pa0[i];
                o[1] = Pb0[i];
              }
              if (t1 < m) {
                int32_t* o = dots + ((int64_t)t1 * n_rows + n) * (k / 16) + jo;
                o[0] = Pa1[i];
                o[1] = Pb1[i];
              }
            }
          }
        } else {
          const int sca = (int)(int8_t)(scs & 0xffu), scb = (int)(int8_t)(scs >> 8);
          const float4 d0 = *reinterpret_cast<const float4*>(s_dx + (bl0 + grp) * kMT + 4 * g);
          const float4 d1 = *reinterpret_cast<const float4*>(s_dx + (bl0 + grp) * kMT + 16 + 4 * g);
          // |sc P| <= 128 * 16 * 127 * 32 per sub-block: the integer sum is
          // exact in int32 and in its fp32 conversion (< 2^24).
          accs0[0] = fmaf(d0.x, (float)(__mul24(Pa0[0], sca) + __mul24(Pb0[0], scb)), accs0[0]);
          accs0[1] = fmaf(d0.y, (float)(__mul24(Pa0[1], sca) + __mul24(Pb0[1], scb)), accs0[1]);
          accs0[2] = fmaf(d0.z, (float)(__mul24(Pa0[2], sca) + __mul24(Pb0[2], scb)), accs0[2]);
          accs0[3] = fmaf(d0.w, (float)(__mul24(Pa0[3], sca) + __mul24(Pb0[3], scb)), accs0[3]);
          accs1[0] = fmaf(d1.x, (float)(__mul24(Pa1[0], sca) + __mul24(Pb1[0], scb)), accs1[0]);
          accs1[1] = fmaf(d1.y, (float)(__mul24(Pa1[1], sca) + __mul24(Pb1[1], scb)), accs1[1]);
          accs1[2] = fmaf(d1.z, (float)(__mul24(Pa1[2], sca) + __mul24(Pb1[2], scb)), accs1[2]);
          accs1[3] = fmaf(d1.w, (float)(__mul24(Pa1[3], sca) + __mul24(Pb1[3], scb)), accs1[3]);
        }
      }
      if constexpr (!DOTS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc0[i] = fmaf(d, accs0[i], acc0[i]);
          acc1[i] = fmaf(d, accs1[i], acc1[i]);
        }
      }
    }
    // The weights two ahead, requested once this super-block's products
    // are done (Q6_K 4096 x 12288: 22.6 -> 21.9 us per kernel; Q4_K the same).
    issue(buf, sb + 2);
    };
  for (int sb = sb_begin; sb < sb_end; sb += 2) {
    step(sb, bufA);
    if (sb + 1 < sb_end) step(sb + 1, bufB);
  }

  if constexpr (!DOTS) {
    // The waves' sums, added in wave order through LDS.
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);  // [NW][8][64]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[(wid * 8 + i) * 64 + lane] = acc0[i];
      red[(wid * 8 + 4 + i) * 64 + lane] = acc1[i];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < 8 * 64; o += NW * 64) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[w * 8 * 64 + o];
      const int i = o >> 6, l = o & 63;
      const int tt = (i < 4 ? 0 : 16) + 4 * (l >> 4) + (i & 3);
      const int64_t nn = row0 + (l & 15);
      if (tt < m && nn < n_rows) y[(int64_t)tt * n_rows + nn] = s;
    }
  }
}

bool shape_ok(int fmt, int64_t n, int64_t k, int m) {
  // Buffer offsets are 32-bit: a tile's rows and the tiled activations must fit.
  const int64_t rb = (k / 256) * (fmt == kQ4_K ? 144 : 210);
  return (fmt == kQ4_K || fmt == kQ6_K) && m >= 1 && m <= kMT && k >= 256 && k % 256 == 0 && n >= 1 &&
         rb * kRows < (1ll << 30) && (k / 32) * kMT * 32 < (1ll << 30);
}

// Waves per workgroup: enough to keep about 16 waves per CU (four per
// SIMD) when the row tiles alone do not, each wave taking at least two
// super-blocks; at most 16, which leaves 128 registers per lane: the Q4_K
// and Q6_K instances need 118 and 126. Measured: Q4_K 12288 x 4096 with 8
// waves (target 16 against 12) kernel 16.9 -> 16.55 us; Q6_K 4096 x 12288
// with 16 waves against 8, call 26.7 -> 26.4 us (an earlier version of the
// kernel spilled at 16 waves: 27.6 against 25.9 us).
int waves_for(int64_t n, int64_t k) {
  const int64_t tiles = (n + kRows - 1) / kRows;
  const int64_t want = (int64_t)device_cus() * 16;
  const int nsb = (int)(k / 256);
  int nw = 4;
  while (nw < 16 && tiles * nw < want && nsb / (nw * 2) >= 2) nw *= 2;
  return nw;
}

template <int FMT, int NW, bool DOTS>
hipError_t launch_t(const uint8_t* w, const int8_t* xqt, const float* dxt, const float* cxt, float* y,
                    int32_t* dots, int64_t n, int64_t k, int m, hipStream_t s) {
  auto kern = gemm32_kernel<FMT, NW, DOTS>;
  const int nsb = (int)(k / 256);
  const int spw = (nsb + NW - 1) / NW;
  size_t lds = (size_t)NW * WaveLds<FMT>::bytes(spw);
  const size_t red = (size_t)NW * 8 * 64 * sizeof(float);
  if (lds < red) lds = red;
  if (lds > (size_t)kLdsBytes) return hipErrorInvalidValue;
  int per_cu = 0;  // raises the dynamic-LDS limit (once per kernel and device)
  hipError_t qe = kernel_residency(reinterpret_cast<const void*>(kern), NW * 64, lds, true, &per_cu);
  if (qe != hipSuccess) return qe;
  const unsigned tiles = (unsigned)((n + kRows - 1) / kRows);
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(NW * 64), lds, s, w, xqt, dxt, cxt, y, dots, n, k, m, spw);
  return hipGetLastError();
}

template <int FMT, bool DOTS>
hipError_t launch_fmt(const uint8_t* w, const int8_t* xqt, const float* dxt, const float* cxt, float* y,
                      int32_t* dots, int64_t n, int64_t k, int m, hipStream_t s) {
  const int nw = waves_for(n, k);
  if (nw == 4) return launch_t<FMT, 4, DOTS>(w, xqt, dxt, cxt, y, dots, n, k, m, s);
  if (nw == 16) return launch_t<FMT, 16, DOTS>(w, xqt, dxt, cxt, y, dots, n, k, m, s);
  return launch_t<FMT, 8, DOTS>(w, xqt, dxt, cxt, y, dots, n, k, m, s);
}

}  // namespace

bool mfma_supported(int fmt) { return fmt == kQ4_K || fmt == kQ6_K; }

size_t gemm32_tiled_act_bytes(int64_t k) { return (size_t)(k / 32) * kMT * 32; }

hipError_t launch_gemm32(int fmt, const uint8_t* w, const int8_t* xqt, const float* dxt, const float* cxt,
                         float* y, int64_t n, int64_t k, int m, hipStream_t s) {
  if (!shape_ok(fmt, n, k, m)) return hipErrorInvalidValue;
  return fmt == kQ4_K ? launch_fmt<kQ4_K, false>(w, xqt, dxt, cxt, y, nullptr, n, k, m, s)
                      : launch_fmt<kQ6_K, false>(w, xqt, dxt, cxt, y, nullptr, n, k, m, s);
}

hipError_t launch_gemm32_dots(int fmt, const uint8_t* w, const int8_t* xqt, int32_t* dots, int64_t n,
                              int64_t k, int m, hipStream_t s) {
  if (!shape_ok(fmt, n, k, m)) return hipErrorInvalidValue;
  return fmt == kQ4_K ? launch_fmt<kQ4_K, true>(w, xqt, nullptr, nullptr, nullptr, dots, n, k, m, s)
                      : launch_fmt<kQ6_K, true>(w, xqt, nullptr, nullptr, nullptr, dots, n, k, m, s);
}

}  // namespace qg
