// Decode attention of one new token over an fp16 KV cache, in two stages.
//
// The long-context attention of "Why expert caching can't save dense models:
// running a 27B dense model in 16 GB VRAM" (xhh.club, in-place compute and
// single-stream fusion section and its Q&A) splits the cached tokens into
// chunks, computes each chunk's partial softmax result, then merges the
// chunks; a short context takes one online-softmax pass. Here:
//
// Stage 1 (attn_partial_kernel): one workgroup per (chunk, key/value head)
// computes, for the G query heads that share that key/value head
// (grouped-query attention; the workload shape, 16 query heads over 2
// key/value heads of dimension 256, is the gated-attention shape in
// "Understanding Qwen3.6-35B-A3B in llama.cpp", cnblogs, section 1.1), the
// chunk's running maximum m, sum l of exp(s - m) and unnormalised output
// sum_t exp(s_t - m) v_t. Keys and values are read once per group of G
// heads. A token's row of D fp16 values is spread over D/8 lanes, 16 bytes
// each, so one 128-bit load instruction of a wave reads 1 KB of consecutive
// tokens; the lanes of a token add their partial dot products with DPP adds
// and one cross-row swap, and each lane keeps the running state for its 8
// dimensions. Scores are kept in base 2 (q pre-scaled by log2(e)/sqrt(D)),
// so every exponential is one v_exp_f32, and the running maximum is a lazy
// reference (moved only when a score exceeds it by 2^8), so most tokens cost
// one exponential per head and no rescaling.
//
// Stage 2 (attn_merge_kernel): per query head, M = max_c m_c,
// L = sum_c l_c 2^(m_c - M), o = sum_c 2^(m_c - M) o_c / L, with the
// dimensions split over workgroups and the chunks over four waves.
//
// With a single chunk stage 1 normalises and writes o itself.
#include "attn.h"
#include "common.cuh"
#include "internal.h"

namespace qg {

namespace {

#ifndef QG_ATTN_MFMA
#define QG_ATTN_MFMA 0  // 1: scores on matrix cores for head dimension 256 with 8 query heads per key/value head (measured slower)
#endif

constexpr int kAttnWaves = 4;
#ifndef QG_ATTN_WGS_PER_CU
#define QG_ATTN_WGS_PER_CU 1  // stage-1 workgroups per CU the chunking aims for (measured: 1 beats 2, 3, 4)
#endif
#ifndef QG_ATTN_MIN_BATCHES
#define QG_ATTN_MIN_BATCHES 2  // shortest chunk, in batched iterations of the workgroup
#endif
#ifndef QG_ATTN_BATCH
#define QG_ATTN_BATCH 2
#endif
constexpr int kAttnBatch = QG_ATTN_BATCH;  // token iterations whose loads are issued together (double-buffered)
constexpr int kBufWord3 = 0x00020000;  // raw buffer resource, gfx9 family

QG_DEV float h2f(uint32_t bits) { return half_bits(bits & 0xffffu); }

// How far (base 2) a score may exceed a head's reference maximum before the
// running sums are rescaled to a new maximum.
constexpr float kTau = 8.0f;

template <int CTRL>
QG_DEV float dppf(float v) {  // bound_ctrl set: every lane's partner exists, lets the add take the DPP operand
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
// Sum over each row of 16 lanes, in every lane of the row: quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
QG_DEV float row_sum16(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  return v + dppf<0x140>(v);
}
// Rows 2i and 2i+1 hold row sums; every lane of both gets their total
// (v_permlane16_swap exchanges the odd rows of one copy with the even rows of
// the other, so the two results hold row 2i and row 2i+1 in every lane).
QG_DEV float pair_rows_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Running softmax state of one lane for G heads and its 8 dimensions.
template <int G>
struct AState {
  float m[G], l[G], acc[G][8];
};

// One row of the merge buffer: the 8-dimension sums of every lane at 0 .. D-1
// (16-byte aligned for 128-bit LDS accesses), then m and l.
template <int D>
constexpr int kRedRow = D + 4;

// Combine the states of the two halves of the lane set that a lane swap
// pairs up (the permlane call returns both partners' values in every lane).
template <int G, bool ROWS16>
QG_DEV void swap_merge(AState<G>& st) {
  auto sw = [](float v) __attribute__((always_inline)) {
    if constexpr (ROWS16) return __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    else return __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  };
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const auto mm = sw(st.m[j]);
    const auto ll = sw(st.l[j]);
    const float ma = __uint_as_float(mm[0]), mb = __uint_as_float(mm[1]);
    const float M = fmaxf(ma, mb);
    const float ca = ma == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ma - M);
    const float cb = mb == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mb - M);
    st.m[j] = M;
    st.l[j] = __uint_as_float(ll[0]) * ca + __uint_as_float(ll[1]) * cb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const auto aa = sw(st.acc[j][i]);
      st.acc[j][i] = __uint_as_float(aa[0]) * ca + __uint_as_float(aa[1]) * cb;
    }
  }
}

// Merge the per-lane states of a workgroup in a fixed order and write the
// chunk's partial (or, for a single chunk, the normalised output). Lane
// (slot, dl) holds dimensions 8 dl .. 8 dl + 7 of every head of its group.
// First the token slots of each wave: with two slots (32-lane halves) one
// cross-half swap per value; with four (16-lane rows) a row swap, then the
// half swap, so every slot ends up with the wave's total. Then each wave
// stores its state in LDS and the G heads are spread over the workgroup's
// slots: the slot that owns head j merges waves 0, 1, 2, 3 in that order.
template <int D, int G>
QG_DEV void attn_finish(AState<G>& st, float (&red)[kAttnWaves][G][kRedRow<D>], int wid, int lane, int c,
                        int kvh, int nchunks, float* __restrict__ out, float* __restrict__ pm,
                        float* __restrict__ pl, float* __restrict__ po) {
  constexpr int LPT = D / 8;
  constexpr int TPW = 64 / LPT;
  static_assert(TPW == 2 || TPW == 4, "token slots per wave");
  const int dl = lane % LPT;
  const int slot = lane / LPT;
  if constexpr (TPW == 4) swap_merge<G, true>(st);
  swap_merge<G, false>(st);
  if (slot == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (dl == 0) {
        red[wid][j][D] = st.m[j];
        red[wid][j][D + 1] = st.l[j];
      }
      float4* r = reinterpret_cast<float4*>(&red[wid][j][8 * dl]);
      r[0] = make_float4(st.acc[j][0], st.acc[j][1], st.acc[j][2], st.acc[j][3]);
      r[1] = make_float4(st.acc[j][4], st.acc[j][5], st.acc[j][6], st.acc[j][7]);
    }
  }
  __syncthreads();
  constexpr int kOwners = kAttnWaves * TPW;
#pragma unroll 1
  for (int j = wid * TPW + slot; j < G; j += kOwners) {
    float m = red[0][j][D], l = red[0][j][D + 1];
    float a[8];
    {
      const float4* r = reinterpret_cast<const float4*>(&red[0][j][8 * dl]);
      const float4 u = r[0], v = r[1];
      a[0] = u.x, a[1] = u.y, a[2] = u.z, a[3] = u.w, a[4] = v.x, a[5] = v.y, a[6] = v.z, a[7] = v.w;
    }
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) {
      const float mb = red[w][j][D], lb = red[w][j][D + 1];
      const float4* r = reinterpret_cast<const float4*>(&red[w][j][8 * dl]);
      const float4 u = r[0], v = r[1];
      const float b[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
      const float M = fmaxf(m, mb);
      const float ca = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      const float cb = mb == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mb - M);
      m = M;
      l = l * ca + lb * cb;
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = a[i] * ca + b[i] * cb;
    }
    const int64_t h = (int64_t)kvh * G + j;
    if (nchunks == 1) {
      const float inv = 1.0f / l;
      float4* op = reinterpret_cast<float4*>(out + h * D + 8 * dl);
      op[0] = make_float4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
      op[1] = make_float4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv);
    } else {
      if (dl == 0) {
        pm[h * nchunks + c] = m;
        pl[h * nchunks + c] = l;
      }
      float4* op = reinterpret_cast<float4*>(po + (h * nchunks + c) * D + 8 * dl);
      op[0] = make_float4(a[0], a[1], a[2], a[3]);
      op[1] = make_float4(a[4], a[5], a[6], a[7]);
    }
  }
}

// D: head dimension (128 or 256); G: query heads per key/value head.
// grid = (nchunks, n_kv); block = 4 waves.
template <int D, int G>
__global__ __launch_bounds__(kAttnWaves * 64, 2) void attn_partial_kernel(
    const float* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    float* __restrict__ out, float* __restrict__ pm, float* __restrict__ pl, float* __restrict__ po,
    int64_t n_ctx, int64_t chunk, int nchunks, float qscale) {
  constexpr int LPT = D / 8;          // lanes per token
  constexpr int TPW = 64 / LPT;       // tokens per wave load
  __shared__ __align__(16) float red[kAttnWaves][G][kRedRow<D>];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = blockIdx.x;
  const int kvh = blockIdx.y;
  const int dl = lane % LPT;          // this lane's 8 dimensions: 8 dl .. 8 dl + 7
  const int slot = lane / LPT;        // token slot within a wave load

  // Query rows of the group, this lane's dimensions (scaled below, once the
  // first K/V batches have been requested, so the latencies overlap).
  float4 qa[G], qb[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float4* qp = reinterpret_cast<const float4*>(q + ((int64_t)kvh * G + j) * D + 8 * dl);
    qa[j] = qp[0];
    qb[j] = qp[1];
  }
  float qr[G][8];

  AState<G> st;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = -INFINITY;
    st.l[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[j][i] = 0.0f;
  }

  // This head's cache through buffer resources spanning exactly its n_ctx
  // rows: reads past the last token return zeros without a memory access.
  const int64_t head_off = (int64_t)kvh * n_ctx * D;
  const int nbytes = (int)(n_ctx * D * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + head_off), 0, nbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + head_off), 0, nbytes, kBufWord3);

  const int64_t t0 = (int64_t)c * chunk;
  const int64_t t1 = (t0 + chunk) < n_ctx ? (t0 + chunk) : n_ctx;
  constexpr int kStep = kAttnWaves * TPW;  // tokens per iteration of the whole workgroup

  // One token per lane group: scores of the G heads (sum over the LPT lanes
  // of the token), then the lazily rescaled online softmax: the reference
  // maximum m of a head only moves when a score exceeds it by more than
  // kTau (base 2), so the common step is e = 2^(s - m), l += e,
  // acc += e * v, and the rescale is a rare wave-uniform branch.
  auto token = [&](const u32x4& kb, const u32x4& vb, bool valid) __attribute__((always_inline)) {
    const uint32_t kw[4] = {kb.x, kb.y, kb.z, kb.w};
    const uint32_t vw[4] = {vb.x, vb.y, vb.z, vb.w};
    float kf[8], vf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kf[2 * i] = h2f(kw[i]);
      kf[2 * i + 1] = h2f(kw[i] >> 16);
      vf[2 * i] = h2f(vw[i]);
      vf[2 * i + 1] = h2f(vw[i] >> 16);
    }
    float sc[G];
    bool big = false;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float x = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) x = fmaf(qr[j][i], kf[i], x);
      x = row_sum16(x);
      if constexpr (LPT == 32) x = pair_rows_sum(x);
      sc[j] = valid ? x : -INFINITY;
      big |= sc[j] > st.m[j] + kTau;  // m = -inf: any valid score
    }
    if (__builtin_amdgcn_ballot_w64(big)) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float mn = fmaxf(st.m[j], sc[j]);
        const float cr = mn == st.m[j] ? 1.0f : __builtin_amdgcn_exp2f(st.m[j] - mn);  // exp2(-inf) = 0
        st.m[j] = mn;
        st.l[j] *= cr;
#pragma unroll
        for (int i = 0; i < 8; ++i) st.acc[j][i] *= cr;
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float e = valid ? __builtin_amdgcn_exp2f(sc[j] - st.m[j]) : 0.0f;
      st.l[j] += e;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.acc[j][i] = fmaf(e, vf[i], st.acc[j][i]);
    }
  };

  // Batches of kAttnBatch token loads per lane, double-buffered: the next
  // batch is requested before the current one is processed.
  auto fetch = [&](u32x4 (&kb)[kAttnBatch], u32x4 (&vb)[kAttnBatch], int64_t tb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kAttnBatch; ++u) {
      const int64_t t = tb + (int64_t)u * kStep + slot;
      const int off = (int)((t < t1 ? t : n_ctx) * (D * 2)) + 16 * dl;  // past the chunk: out of range, zeros
      kb[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 2);
      vb[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 2);
    }
  };
  auto consume = [&](const u32x4 (&kb)[kAttnBatch], const u32x4 (&vb)[kAttnBatch], int64_t tb)
                     __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kAttnBatch; ++u) token(kb[u], vb[u], tb + (int64_t)u * kStep + slot < t1);
  };
  constexpr int64_t kBatchTokens = (int64_t)kStep * kAttnBatch;
  u32x4 kA[kAttnBatch], vA[kAttnBatch], kB[kAttnBatch], vB[kAttnBatch];
  int64_t tb = t0 + (int64_t)wid * TPW;
  if (tb < t1) fetch(kA, vA, tb);
  if (tb + kBatchTokens < t1) fetch(kB, vB, tb + kBatchTokens);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float4 a = qa[j], b = qb[j];
    qr[j][0] = a.x * qscale; qr[j][1] = a.y * qscale; qr[j][2] = a.z * qscale; qr[j][3] = a.w * qscale;
    qr[j][4] = b.x * qscale; qr[j][5] = b.y * qscale; qr[j][6] = b.z * qscale; qr[j][7] = b.w * qscale;
  }
  // Two batches in flight: each buffer is refilled with the batch after
  // next as soon as it has been consumed.
  while (tb < t1) {
    consume(kA, vA, tb);
    if (tb + 2 * kBatchTokens < t1) fetch(kA, vA, tb + 2 * kBatchTokens);
    tb += kBatchTokens;
    if (tb >= t1) break;
    consume(kB, vB, tb);
    if (tb + 2 * kBatchTokens < t1) fetch(kB, vB, tb + 2 * kBatchTokens);
    tb += kBatchTokens;
  }

  attn_finish<D, G>(st, red, wid, lane, c, kvh, nchunks, out, pm, pl, po);
}

typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Stage 1 with the scores on matrix cores, for D = 256 and G = 8 (the
// workload shape). Per wave and tile of 16 tokens, S^T[16 tokens x 16 heads]
// = K_tile . Q^T is v_mfma_f32_16x16x16_f16 over 16 steps of 4 dimensions
// (heads 8..15 are zero padding): the A operand is the lane's token row
// (lane = token + 16 g reads bytes 128 g .. 128 g + 127 of its row, so step
// s covers dimensions 64 g + 4 s .. + 3), the B operand the query with the
// same dimension mapping. The fp32 query is split into fp16 halves
// hi + lo (scaled per head by a power of two that keeps both normal and
// finite), so two MFMAs per step give the scores to about 2^-22 relative;
// keys are exact in fp16 and products accumulate in fp32. The output lane
// (head h = lane % 16, tokens 4 (lane / 16) + r) then runs the lazily
// rescaled softmax for its head, the weights go through a small LDS table,
// and P.V runs on the VALU in the layout of the other kernel (lane = token
// slot x 8 dimensions, all 8 heads).
__global__ __launch_bounds__(kAttnWaves * 64, 2) void attn_partial_mfma_kernel(
    const float* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    float* __restrict__ out, float* __restrict__ pm, float* __restrict__ pl, float* __restrict__ po,
    int64_t n_ctx, int64_t chunk, int nchunks, float qscale) {
  constexpr int D = 256, G = 8;
  __shared__ __align__(16) float red[kAttnWaves][G][kRedRow<D>];
  __shared__ float pbuf[kAttnWaves][16][G];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = blockIdx.x;
  const int kvh = blockIdx.y;
  const int dl = lane & 31;   // P.V layout: dimensions 8 dl .. 8 dl + 7
  const int slot = lane >> 5;  // P.V layout: token slot
  const int mh = lane & 15;   // MFMA layout: token row (A) or head column (B, D)
  const int mg = lane >> 4;   // MFMA layout: group of 4 in the reduction / output rows

  // Query operand: head mh (zero for mh >= G), dimensions 64 mg + 4 s + e.
  // Scale: q * qscale * 2^e with 2^e chosen per head so its largest value
  // lands in [2^13, 2^14): both fp16 halves stay normal and finite.
  float qv[64];
  float qmax = 0.0f;
  if (mh < G) {
    const float4* qp = reinterpret_cast<const float4*>(q + ((int64_t)kvh * G + mh) * D + 64 * mg);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 v = qp[i];
      qv[4 * i] = v.x * qscale; qv[4 * i + 1] = v.y * qscale; qv[4 * i + 2] = v.z * qscale; qv[4 * i + 3] = v.w * qscale;
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) qmax = fmaxf(qmax, fabsf(qv[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) qv[i] = 0.0f;
  }
  qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
  int qe = 0;
  if (qmax > 0.0f) {
    (void)frexpf(qmax, &qe);  // qmax in [2^(qe-1), 2^qe)
    qe = 14 - qe;
  }
  const float up = ldexpf(1.0f, qe), down = ldexpf(1.0f, -qe);
  h16x4 qh[16], ql[16];
#pragma unroll
  for (int st = 0; st < 16; ++st)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = qv[4 * st + e] * up;
      const _Float16 hi = (_Float16)v;
      qh[st][e] = hi;
      ql[st][e] = (_Float16)(v - (float)hi);
    }

  AState<G> st;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = -INFINITY;
    st.l[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[j][i] = 0.0f;
  }
  float m = -INFINITY;   // reference maximum of head mh (same in its four lanes)
  float lsum = 0.0f;     // this lane's share of head mh's sum of weights

  const int64_t head_off = (int64_t)kvh * n_ctx * D;
  const int nbytes = (int)(n_ctx * D * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + head_off), 0, nbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + head_off), 0, nbytes, kBufWord3);
  const int64_t t0 = (int64_t)c * chunk;
  const int64_t t1 = (t0 + chunk) < n_ctx ? (t0 + chunk) : n_ctx;

  // K rows for the MFMA (past the chunk: out of range, zeros) and V rows for
  // P.V. The next tile's K is requested right after this tile's MFMAs and
  // each V register set is refilled as soon as P.V has used it, so a tile's
  // loads are in flight while the previous tile is processed.
  u32x4 kr[8], vr[8];
  auto load_k = [&](int64_t tb) __attribute__((always_inline)) {
    const int64_t tk = tb + mh;
    const int koff = (int)((tk < t1 ? tk : n_ctx) * (D * 2)) + 128 * mg;
#pragma unroll
    for (int u = 0; u < 8; ++u) kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 16 * u, 0, 2);
  };
  auto load_v = [&](int64_t tb, int it) __attribute__((always_inline)) {
    const int64_t tv = tb + 2 * it + slot;
    const int voff = (int)((tv < t1 ? tv : n_ctx) * (D * 2)) + 16 * dl;
    vr[it] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 2);
  };
  {
    const int64_t tb = t0 + 16 * (int64_t)wid;
    load_k(tb);
#pragma unroll
    for (int it = 0; it < 8; ++it) load_v(tb, it);
  }
  for (int64_t tb = t0 + 16 * (int64_t)wid; tb < t1; tb += 16 * kAttnWaves) {
    const int64_t tn = tb + 16 * kAttnWaves;  // next tile (past t1: no memory traffic)
    f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const u32x2 lo = kr[u].xy, hi = kr[u].zw;
      const h16x4 a0 = __builtin_bit_cast(h16x4, lo), a1 = __builtin_bit_cast(h16x4, hi);
      sc = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, qh[2 * u], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, ql[2 * u], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, qh[2 * u + 1], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, ql[2 * u + 1], sc, 0, 0, 0);
    }
    load_k(tn);
    // Scores of head mh for tokens tb + 4 mg + r.
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = (tb + 4 * mg + r < t1) ? sc[r] * down : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool big = mh < G && mx > m + kTau;
    if (__builtin_amdgcn_ballot_w64(big)) {  // wave-uniform
      const float mn = fmaxf(m, mx);
      const float cr = mn == m ? 1.0f : __builtin_amdgcn_exp2f(m - mn);  // m = -inf: 0
      m = mn;
      lsum *= cr;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float cj = readlane_f(cr, j);  // head j's factor (lane j holds head j)
#pragma unroll
        for (int i = 0; i < 8; ++i) st.acc[j][i] *= cj;
      }
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = sv[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sv[r] - m);
      lsum += p[r];
    }
    if (mh < G) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pbuf[wid][4 * mg + r][mh] = p[r];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's weights are in LDS
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const float4* pp = reinterpret_cast<const float4*>(&pbuf[wid][2 * it + slot][0]);
      const float4 pa = pp[0], pb = pp[1];
      const float pj[G] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
      const uint32_t vw[4] = {vr[it].x, vr[it].y, vr[it].z, vr[it].w};
      float vf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vf[2 * i] = h2f(vw[i]);
        vf[2 * i + 1] = h2f(vw[i] >> 16);
      }
      load_v(tn, it);
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) st.acc[j][i] = fmaf(pj[j], vf[i], st.acc[j][i]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next tile overwrites the table
  }

  // Head sums over the four lanes of each head, then the state in the P.V
  // layout: every lane gets the heads' maxima; slot 0 carries the sums.
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = readlane_f(m, j);
    st.l[j] = slot == 0 ? readlane_f(lsum, j) : 0.0f;
  }
  attn_finish<D, G>(st, red, wid, lane, c, kvh, nchunks, out, pm, pl, po);
}

// grid = (n_heads, D / 64); block = 4 waves. The chunk maxima and sums are
// read with vector loads by all threads: M = max_c m_c and the chunk weights
// w_c = 2^(m_c - M) go to LDS, L = sum_c w_c l_c. Then wave g adds
// w_c o_c[d] over chunks c = g, g + 4, ... for the 64 dimensions of this
// block (one per lane, up to 16 loads in flight), and wave 0 adds the four
// sums in wave order.
constexpr int kMergeWaves = 4;
#ifndef QG_MERGE_UNROLL
#define QG_MERGE_UNROLL 32
#endif
constexpr int kMergeUnroll = QG_MERGE_UNROLL;  // partial outputs a merge wave loads per pass
constexpr int kMaxChunks = 1024;

QG_DEV float block_reduce(float v, float* sh, bool is_max) {
  // every thread gets the result; sh holds kMergeWaves floats
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kMergeWaves; ++i) r = is_max ? fmaxf(r, sh[i]) : r + sh[i];
  return r;
}

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void attn_merge_kernel(const float* __restrict__ pm,
                                                                    const float* __restrict__ pl,
                                                                    const float* __restrict__ po,
                                                                    float* __restrict__ out, int nchunks) {
  __shared__ float wts[kMaxChunks];
  __shared__ float red[kMergeWaves][64];
  __shared__ float sh[kMergeWaves];
  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const float* m = pm + h * nchunks;
  const float* l = pl + h * nchunks;
  const int d = blockIdx.y * 64 + lane;
  const float* o = po + h * nchunks * D + d;
  // Every load of the first pass is issued up front: the chunk maxima and
  // sums of this thread's first chunk and the wave's first kMergeUnroll
  // partial outputs (they do not depend on the weights), so their latencies
  // overlap instead of following each other.
  const float m0 = tid < nchunks ? m[tid] : -INFINITY;
  const float l0 = tid < nchunks ? l[tid] : 0.0f;
  float x[kMergeUnroll];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const int c = w + u * kMergeWaves;
    x[u] = c < nchunks ? o[(int64_t)c * D] : 0.0f;
  }
  float M = m0;
  for (int c = tid + kMergeWaves * 64; c < nchunks; c += kMergeWaves * 64) M = fmaxf(M, m[c]);
  M = block_reduce(M, sh, true);
  float Lp = 0.0f;
  if (tid < nchunks) {
    const float wt = m0 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m0 - M);
    wts[tid] = wt;
    Lp = l0 * wt;
  }
  for (int c = tid + kMergeWaves * 64; c < nchunks; c += kMergeWaves * 64) {
    const float wt = m[c] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[c] - M);
    wts[c] = wt;
    Lp = fmaf(l[c], wt, Lp);
  }
  const float L = block_reduce(Lp, sh, false);  // its barriers also publish wts
  float acc = 0.0f;
  for (int c0 = w;;) {
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int c = c0 + u * kMergeWaves;
      if (c < nchunks) acc = fmaf(x[u], wts[c], acc);
    }
    c0 += kMergeWaves * kMergeUnroll;
    if (c0 >= nchunks) break;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int c = c0 + u * kMergeWaves;
      x[u] = c < nchunks ? o[(int64_t)c * D] : 0.0f;
    }
  }
  red[w][lane] = acc;
  __syncthreads();
  if (w != 0) return;
  float oo = red[0][lane];
#pragma unroll
  for (int v = 1; v < kMergeWaves; ++v) oo += red[v][lane];
  out[h * D + d] = oo / L;
}

template <int D, int G>
hipError_t launch_dg(const AttnShape& a, const AttnPlan& pl, const float* q, const uint16_t* k, const uint16_t* v,
                     float* out, void* ws, hipStream_t s) {
  const float qscale = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(D)
  float* pm = nullptr;
  float* plv = nullptr;
  float* po = nullptr;
  if (pl.nchunks > 1) {  // workspace: o partials [n_heads, nchunks, D], then m and l [n_heads, nchunks]
    po = static_cast<float*>(ws);
    pm = po + (int64_t)a.n_heads * pl.nchunks * D;
    plv = pm + (int64_t)a.n_heads * pl.nchunks;
  }
  if (attn_uses_mfma(a))
    hipLaunchKernelGGL(attn_partial_mfma_kernel, dim3((unsigned)pl.nchunks, (unsigned)a.n_kv),
                       dim3(kAttnWaves * 64), 0, s, q, k, v, out, pm, plv, po, a.n_ctx, pl.chunk,
                       (int)pl.nchunks, qscale);
  else
    hipLaunchKernelGGL((attn_partial_kernel<D, G>), dim3((unsigned)pl.nchunks, (unsigned)a.n_kv),
                       dim3(kAttnWaves * 64), 0, s, q, k, v, out, pm, plv, po, a.n_ctx, pl.chunk,
                       (int)pl.nchunks, qscale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nchunks == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel<D>, dim3((unsigned)a.n_heads, D / 64), dim3(kMergeWaves * 64), 0, s, pm,
                     plv, po, out, (int)pl.nchunks);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnShape& a, const AttnPlan& pl, const float* q, const uint16_t* k, const uint16_t* v,
                    float* out, void* ws, hipStream_t s) {
  switch (a.n_heads / a.n_kv) {
    case 1: return launch_dg<D, 1>(a, pl, q, k, v, out, ws, s);
    case 2: return launch_dg<D, 2>(a, pl, q, k, v, out, ws, s);
    case 4: return launch_dg<D, 4>(a, pl, q, k, v, out, ws, s);
    case 8: return launch_dg<D, 8>(a, pl, q, k, v, out, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attn_uses_mfma(const AttnShape& a) {
  return QG_ATTN_MFMA && a.head_dim == 256 && a.n_heads == 8 * a.n_kv;
}

bool attn_supported(const AttnShape& a) {
  if (a.head_dim != 128 && a.head_dim != 256) return false;
  if (a.n_kv < 1 || a.n_heads < a.n_kv || a.n_heads % a.n_kv) return false;
  const int g = a.n_heads / a.n_kv;
  if (g != 1 && g != 2 && g != 4 && g != 8) return false;
  if (a.n_kv > 65535) return false;
  // Byte offsets inside one head's cache are 32-bit.
  return a.n_ctx >= 1 && a.n_ctx * a.head_dim * 2 + 4096 < ((int64_t)1 << 31);
}

AttnPlan attn_plan(const AttnShape& a) {
  // Tokens one workgroup iteration covers; a chunk is a whole number of them.
  const bool mf = attn_uses_mfma(a);
  const int64_t step = mf ? (int64_t)kAttnWaves * 16 : (int64_t)kAttnWaves * (64 / (a.head_dim / 8));
  const int64_t min_chunk = mf ? step : step * kAttnBatch * QG_ATTN_MIN_BATCHES;
  // Enough chunks for QG_ATTN_WGS_PER_CU workgroups per CU (at most kMaxChunks), none
  // shorter than QG_ATTN_MIN_BATCHES batched iterations of the workgroup.
  int64_t want = ((int64_t)device_cus() * QG_ATTN_WGS_PER_CU + a.n_kv - 1) / a.n_kv;
  if (want > kMaxChunks) want = kMaxChunks;
  int64_t nch = (a.n_ctx + min_chunk - 1) / min_chunk;
  if (nch > want) nch = want;
  if (nch < 1) nch = 1;
  int64_t chunk = (a.n_ctx + nch - 1) / nch;
  chunk = (chunk + step - 1) / step * step;
  AttnPlan p;
  p.chunk = chunk;
  p.nchunks = (a.n_ctx + chunk - 1) / chunk;
  return p;
}

size_t attn_workspace_bytes(const AttnShape& a) {
  const AttnPlan p = attn_plan(a);
  if (p.nchunks <= 1) return 0;
  return (size_t)a.n_heads * (size_t)p.nchunks * (2 + (size_t)a.head_dim) * sizeof(float);
}

hipError_t launch_attn(const AttnShape& a, const float* q, const uint16_t* k, const uint16_t* v, float* out,
                       void* ws, hipStream_t s) {
  if (!attn_supported(a)) return hipErrorInvalidValue;
  const AttnPlan p = attn_plan(a);
  return a.head_dim == 128 ? launch_d<128>(a, p, q, k, v, out, ws, s) : launch_d<256>(a, p, q, k, v, out, ws, s);
}

}  // namespace qg
