// MoE FFN layer on the device: router, top-k + softmax, expert grouping,
// grouped expert GEMVs, SwiGLU re-quantization and the weighted combine.
//
// A router scores the experts for each token and only the selected experts
// run; the model shape is hidden 2048, 256 experts with 8 routed plus one
// shared expert active, expert intermediate 512 ("Understanding
// Qwen3.6-35B-A3B in llama.cpp", cnblogs, section 1.1). Router, top-k,
// softmax and the expert gate/up, SwiGLU, down and weighted aggregation all
// run on the GPU so the selected experts never travel to the host ("01 ·
// Phase overview: from 2B to 8B to MoE", icman.com.cn, stage three and
// ledger items ⑩ and ⑪).
//
// Launch sequence on one stream (no host synchronisation):
//   router_kernel     logits[t, e] = W_r[e] . x[t] (fp32, unquantized x);
//                     the same workgroups quantize x to Q8 (or 16-bit) blocks
// then, when the shapes fit it, the two-launch expert stage of moe_fused.hip
// (routing + gate|up + SwiGLU + requant, then down + combine); otherwise:
//   route_kernel      top-k per token (ties to the lower index), softmax over
//                     the selected logits, then a table that groups the
//                     (token, slot) pairs by expert so each selected expert's
//                     weights are read once for all tokens that chose it
//   grouped GEMV      gate|up of every used expert and of the shared expert
//   swiglu_q8         h = silu(g) * u per (token, slot), re-quantized
//   grouped GEMV      down of every used expert and of the shared expert
//   combine_kernel    y[t] = sum_k w[t, k] out[t, k] (slot order) + shared
// Slot rows: token t, slot k (k < top_k routed, k == top_k shared) is row
// t * (top_k + 1) + k of the per-slot intermediates.
#include "common.cuh"
#include "internal.h"
#include "moe.h"
#include "route.cuh"
#include "s16.cuh"
#include "s16.h"
#include "swiglu.h"

#ifndef QG_MOE_FUSED
#define QG_MOE_FUSED 1  // expert stage in two launches when the shapes allow it
#endif

namespace qg {

constexpr int kRouterMaxTok = 16;

// A workgroup computes the logits of ET experts for TT tokens: its 256
// threads split the rows into float4 chunks, each thread accumulates its
// chunks of every (expert, token) pair, and the workgroup adds the partial
// sums in a fixed order (DPP within a wave, then the four waves in order), so
// a logit does not depend on the tiling. Tiles of several experts and several
// tokens cut the bytes each workgroup reads (ET rows of W_r plus TT rows of
// x) from 8 KB x (1 + m) to 8 KB x (ET + TT) at hidden 2048. The router's
// workgroups also quantize x to Q8 blocks for the expert GEMVs (block b by
// workgroup b mod grid, eight lanes per block as in the activation
// quantizer), so no separate quantizer launch is needed.
// A thread requests a chunk's weights and x before it multiplies any of them,
// so a chunk costs one memory round trip; two chunks are in flight together.
// Experts and tokens past the end re-read the last one and are not stored.
// S16: x is quantized to 16-bit codes (xq16) instead of Q8 codes (xq), with
// the 16-bit activation quantizer's arithmetic.
template <int ET, int TT, bool S16>
__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ wr,
                                                     const float* __restrict__ x,
                                                     float* __restrict__ logits, int8_t* __restrict__ xq,
                                                     int16_t* __restrict__ xq16,
                                                     float* __restrict__ dx, int32_t* __restrict__ sx,
                                                     int n_experts, int64_t hidden, int m) {
  __shared__ float part[4][ET * TT];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n_eg = (n_experts + ET - 1) / ET;
  const int e0 = (int)(blockIdx.x % n_eg) * ET, t0 = (int)(blockIdx.x / n_eg) * TT;
  const float4* wrow[ET];
  const float4* xrow[TT];
#pragma unroll
  for (int i = 0; i < ET; ++i)
    wrow[i] = reinterpret_cast<const float4*>(wr + (int64_t)(e0 + i < n_experts ? e0 + i : n_experts - 1) * hidden);
#pragma unroll
  for (int t = 0; t < TT; ++t)
    xrow[t] = reinterpret_cast<const float4*>(x + (int64_t)(t0 + t < m ? t0 + t : m - 1) * hidden);
  const int64_t nch = hidden / 4;
  float acc[ET][TT];
#pragma unroll
  for (int i = 0; i < ET; ++i)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[i][t] = 0.0f;
#pragma unroll 2
  for (int64_t c = threadIdx.x; c < nch; c += blockDim.x) {
    float4 w[ET], v[TT];
#pragma unroll
    for (int i = 0; i < ET; ++i) w[i] = wrow[i][c];
#pragma unroll
    for (int t = 0; t < TT; ++t) v[t] = xrow[t][c];
#pragma unroll
    for (int i = 0; i < ET; ++i)
#pragma unroll
      for (int t = 0; t < TT; ++t)
        acc[i][t] = fmaf(w[i].x, v[t].x, fmaf(w[i].y, v[t].y, fmaf(w[i].z, v[t].z, fmaf(w[i].w, v[t].w, acc[i][t]))));
  }
#pragma unroll
  for (int i = 0; i < ET; ++i)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float s = group_sum(acc[i][t], 64);
      if (lane == 0) part[wid][i * TT + t] = s;
    }
  // Q8 (or 16-bit) blocks of x: 32 blocks per workgroup pass, eight lanes each.
  const int64_t nblocks = (int64_t)m * (hidden / 32);
  for (int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3); blk < nblocks;
       blk += (int64_t)gridDim.x * 32) {
    // whole 8-lane groups are in or out together
    const int part8 = threadIdx.x & 7;
    const float4 v = reinterpret_cast<const float4*>(x)[blk * 8 + part8];
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = max8(a);
    const float d = (a > 0.0f) ? a / (S16 ? 32767.0f : 127.0f) : 0.0f;
    int sum;
    if constexpr (S16) {
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
      reinterpret_cast<uint2*>(xq16)[blk * 8 + part8] = packed;
      sum = q0 + q1 + q2 + q3;
    } else {
      const uint32_t packed = q8_pack4(v, d, sum);
      reinterpret_cast<uint32_t*>(xq)[blk * 8 + part8] = packed;
    }
    sum = sum4(sum);
    sum += other_quad(sum);
    if (part8 == 0) {
      dx[blk] = d;
      sx[blk] = sum;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < ET * TT) {
    const int i = threadIdx.x / TT, t = threadIdx.x % TT;
    if (e0 + i < n_experts && t0 + t < m)
      logits[(int64_t)(t0 + t) * n_experts + e0 + i] =
          (part[0][threadIdx.x] + part[1][threadIdx.x]) + (part[2][threadIdx.x] + part[3][threadIdx.x]);
  }
}

template <int ET, int TT>
hipError_t launch_router_t(const MoeCall& c, hipStream_t s) {
  const int grid = (c.n_experts + ET - 1) / ET * ((c.m + TT - 1) / TT);
  if (c.xq16)
    hipLaunchKernelGGL((router_kernel<ET, TT, true>), dim3((unsigned)grid), dim3(256), 0, s, c.router, c.x, c.logits,
                       c.xq, c.xq16, c.dx, c.sx, c.n_experts, c.hidden, c.m);
  else
    hipLaunchKernelGGL((router_kernel<ET, TT, false>), dim3((unsigned)grid), dim3(256), 0, s, c.router, c.x,
                       c.logits, c.xq, c.xq16, c.dx, c.sx, c.n_experts, c.hidden, c.m);
  return hipGetLastError();
}

// Tiles: up to 4 tokens per workgroup, and 2 or 4 experts from 5 tokens on
// (one workgroup per expert tile and token tile).
hipError_t launch_router(const MoeCall& c, hipStream_t s) {
  if (c.m <= 1) return launch_router_t<1, 1>(c, s);
  if (c.m <= 2) return launch_router_t<1, 2>(c, s);
  if (c.m <= 4) return launch_router_t<1, 4>(c, s);
  if (c.m <= 8) return launch_router_t<2, 4>(c, s);
  return launch_router_t<4, 4>(c, s);
}

// One workgroup of 64 * m threads. Wave t selects token t's top_k experts and
// their softmax weights; then the (token, slot) pairs are grouped by expert
// into the table read by the grouped GEMV, in entries of at most
// kGroupTokens tokens (each entry reads its expert's weights once):
//   tbl[0] = number of entries;
//   tbl[1 + e * (2 + kGroupTokens) ...] = {expert, count, slot rows}
// Routed entries come first, ordered by the expert's first occurrence
// (token-major, slot order), tokens ascending; then ceil(m / kGroupTokens)
// entries of the shared expert (expert = -1) covering every token.
// NPL: logits held per lane (experts lane + 64 i), n_experts <= 64 * NPL.
template <int NPL>
__global__ void route_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                             float* __restrict__ wts, int32_t* __restrict__ tbl, int n_experts,
                             int top_k, int m) {
  extern __shared__ int32_t sh[];
  const int tid = threadIdx.x;
  const int t = tid >> 6, lane = tid & 63;
  const int npairs = m * top_k;
  uint32_t* sel = reinterpret_cast<uint32_t*>(sh);  // [n_experts] tokens that chose the expert
  int32_t* ebase = sh + n_experts;                  // [n_experts] first table entry of the expert
  int32_t* s_ids = ebase + n_experts;               // [npairs] expert of pair p = token * top_k + slot
  int32_t* nch = s_ids + npairs;                    // [npairs] entries of the expert at its first pair
  int32_t* scan = nch + npairs;                     // [npairs] exclusive prefix sum of nch
  int32_t* routed = scan + npairs;                  // [1] routed entries in all

  for (int i = tid; i < n_experts; i += blockDim.x) sel[i] = 0u;
  __syncthreads();

  if (t < m) {
    // This lane's logits, loaded once; selection works on registers.
    const float* lg = logits + (int64_t)t * n_experts;
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < n_experts ? lg[e] : 0.0f;
    }
    uint64_t taken = 0;  // bit i: expert lane + 64 i already selected (or absent)
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i >= n_experts) taken |= 1ull << i;
    float my_v = -INFINITY;  // lane k keeps the k-th selection
    int my_i = 0;
    for (int k = 0; k < top_k; ++k) {
      uint64_t best = 0;  // below every real key
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const uint64_t key = route_key(v[i], lane + 64 * i);
        if (!((taken >> i) & 1ull) && key > best) best = key;
      }
      best = wave_max_key(best);
      const int bi = route_key_expert(best);
      if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
      if (lane == k) {
        my_v = route_key_value(best);
        my_i = bi;
      }
    }
    const float v0 = __shfl(my_v, 0, 64);
    const float ez = (lane < top_k) ? expf(my_v - v0) : 0.0f;
    const float den = wave_sum(ez);
    if (lane < top_k) {
      ids[t * top_k + lane] = my_i;
      wts[t * top_k + lane] = ez / den;
      s_ids[t * top_k + lane] = my_i;
      atomicOr(&sel[my_i], 1u << t);  // a token selects an expert at most once
    }
  }
  __syncthreads();

  // Rank of a pair among the expert's tokens (tokens ascending) and, at the
  // expert's first pair, the number of table entries the expert needs.
  for (int p = tid; p < npairs; p += blockDim.x) {
    const uint32_t sm = sel[s_ids[p]];
    const int tt = p / top_k;
    const int r = __popc(sm & ((1u << tt) - 1u));
    nch[p] = r == 0 ? (__popc(sm) + kGroupTokens - 1) / kGroupTokens : 0;
  }
  __syncthreads();
  // Entries in order of the experts' first pairs: exclusive scan of nch by
  // wave 0, four pairs per lane (npairs <= 256).
  if (t == 0) {
    int vals[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = 4 * lane + j;
      vals[j] = idx < npairs ? nch[idx] : 0;
      loc += vals[j];
    }
    int inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    int ex = inc - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = 4 * lane + j;
      if (idx < npairs) scan[idx] = ex;
      ex += vals[j];
    }
    if (lane == 63) routed[0] = inc;
  }
  __syncthreads();
  for (int p = tid; p < npairs; p += blockDim.x)
    if (nch[p] > 0) ebase[s_ids[p]] = scan[p];
  __syncthreads();
  const int tstride = 2 + kGroupTokens;
  for (int p = tid; p < npairs; p += blockDim.x) {
    const int e = s_ids[p];
    const uint32_t sm = sel[e];
    const int tok = p / top_k, k = p - tok * top_k;
    const int r = __popc(sm & ((1u << tok) - 1u));
    int32_t* ent = tbl + 1 + (int64_t)(ebase[e] + r / kGroupTokens) * tstride;
    ent[2 + r % kGroupTokens] = tok * (top_k + 1) + k;
    if (r % kGroupTokens == 0) {
      ent[0] = e;
      const int left = __popc(sm) - r;
      ent[1] = left < kGroupTokens ? left : kGroupTokens;
    }
  }
  if (tid == 0) {
    const int nr = routed[0];
    const int nsh = (m + kGroupTokens - 1) / kGroupTokens;
    for (int c = 0; c < nsh; ++c) {
      int32_t* ent = tbl + 1 + (int64_t)(nr + c) * tstride;
      const int t0 = c * kGroupTokens;
      const int n = (m - t0) < kGroupTokens ? (m - t0) : kGroupTokens;
      ent[0] = -1;
      ent[1] = n;
      for (int j = 0; j < n; ++j) ent[2 + j] = (t0 + j) * (top_k + 1) + top_k;
    }
    tbl[0] = nr + nsh;
  }
}

// y[t, c] = sum_k wts[t, k] * out[t*(K+1)+k, c] + out[t*(K+1)+K, c]
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ out,
                                                      const float* __restrict__ wts,
                                                      float* __restrict__ y, int64_t hidden, int m,
                                                      int top_k) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)m * hidden) return;
  const int64_t t = i / hidden, c = i - t * hidden;
  const float* o = out + t * (top_k + 1) * hidden + c;
  float acc = 0.0f;
  for (int k = 0; k < top_k; ++k) acc = fmaf(wts[t * top_k + k], o[(int64_t)k * hidden], acc);
  y[i] = acc + o[(int64_t)top_k * hidden];
}

// Entries: at most one per (token, slot) pair plus the shared-expert chunks.
static int64_t moe_max_entries(int m, int top_k) { return (int64_t)m * top_k + (m + kGroupTokens - 1) / kGroupTokens; }
int64_t moe_table_ints(int m, int top_k) { return 1 + moe_max_entries(m, top_k) * (2 + kGroupTokens); }

hipError_t launch_moe(const MoeCall& c, hipStream_t s) {
  if (c.m < 1 || c.m > kRouterMaxTok || c.top_k > 16) return hipErrorInvalidValue;
  if (c.n_experts < 1 || c.n_experts > 4096 || c.hidden % 32) return hipErrorInvalidValue;
  // 16-bit codes of x and h (Q4_0 experts): the expert GEMVs read them
  // instead of Q8 codes (their scales and sums take dx/sx and hd/hs).
  const bool s16 = c.xq16 != nullptr;
  if (s16 && (kGroupTokens != 1 || !c.hq16 || !q40_s16_grouped_ok(c.hidden) || !q40_s16_grouped_ok(c.inter)))
    return hipErrorInvalidValue;
  // 1. router logits, and x quantized to Q8 (or 16-bit) blocks
  hipError_t e = launch_router(c, s);
  if (e != hipSuccess) return e;
  if (QG_MOE_FUSED && moe_fused_ok(c)) return launch_moe_fused(c, s);
  // 2. top-k, softmax and grouping
  const int npairs = c.m * c.top_k;
  const size_t lds = (2 * (size_t)c.n_experts + 3 * (size_t)npairs + 1) * 4;
  if (c.n_experts <= 256)
    hipLaunchKernelGGL(route_kernel<4>, dim3(1), dim3(64 * c.m), lds, s, c.logits, c.ids, c.wts, c.tbl,
                       c.n_experts, c.top_k, c.m);
  else if (c.n_experts <= 1024)
    hipLaunchKernelGGL(route_kernel<16>, dim3(1), dim3(64 * c.m), lds, s, c.logits, c.ids, c.wts, c.tbl,
                       c.n_experts, c.top_k, c.m);
  else
    hipLaunchKernelGGL(route_kernel<64>, dim3(1), dim3(64 * c.m), lds, s, c.logits, c.ids, c.wts, c.tbl,
                       c.n_experts, c.top_k, c.m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. gate|up of the used experts and the shared expert, on the codes the
  // router kernel wrote
  const int slots = c.top_k + 1;
  const int maxprob = (int)moe_max_entries(c.m, c.top_k);
  GemvProblem g;
  g.w = c.gu;
  g.w_stride = c.gu_stride;
  g.w_shared = c.gu_shared;
  g.tbl = c.tbl;
  g.tbl_stride = 2 + kGroupTokens;
  g.nprob = maxprob;
  g.act_div = slots;
  g.xq = c.xq;
  g.dx = c.dx;
  g.xs = c.hidden;
  g.y = c.gu_out;
  g.ldy = 2 * c.inter;
  g.n = 2 * c.inter;
  g.k = c.hidden;
  g.m = c.m;
  for (int i = 0; i < 4; ++i) g.cb[i] = c.cb[i];
  S16Grouped a;
  if (s16) {
    a.w = c.gu;
    a.w_stride = c.gu_stride;
    a.w_shared = c.gu_shared;
    a.tbl = c.tbl;
    a.tbl_stride = 2 + kGroupTokens;
    a.nprob = maxprob;
    a.xq = c.xq16;
    a.dx = c.dx;
    a.sx = c.sx;
    a.xs = c.hidden;
    a.act_div = slots;
    a.y = c.gu_out;
    a.ldy = 2 * c.inter;
    a.n = 2 * c.inter;
    a.k = c.hidden;
    if ((e = launch_q40_s16_grouped(a, s)) != hipSuccess) return e;
  } else if ((e = launch_gemv(c.fmt, g, false, s)) != hipSuccess) {
    return e;
  }
  // 4. SwiGLU + re-quantization for every slot row
  e = s16 ? launch_swiglu_s16(c.gu_out, 2 * c.inter, c.h, c.hq16, c.hd, c.hs, (int64_t)c.m * slots, c.inter, s)
          : launch_swiglu_q8(c.gu_out, 2 * c.inter, c.h, c.hq, c.hd, c.hs, (int64_t)c.m * slots, c.inter, s);
  if (e != hipSuccess) return e;
  // 5. down of the used experts and the shared expert
  GemvProblem d = g;
  d.w = c.dn;
  d.w_stride = c.dn_stride;
  d.w_shared = c.dn_shared;
  d.act_div = 1;
  d.xq = c.hq;
  d.dx = c.hd;
  d.xs = c.inter;
  d.y = c.out;
  d.ldy = c.hidden;
  d.n = c.hidden;
  d.k = c.inter;
  if (s16) {
    a.w = c.dn;
    a.w_stride = c.dn_stride;
    a.w_shared = c.dn_shared;
    a.xq = c.hq16;
    a.dx = c.hd;
    a.sx = c.hs;
    a.xs = c.inter;
    a.act_div = 1;
    a.y = c.out;
    a.ldy = c.hidden;
    a.n = c.hidden;
    a.k = c.inter;
    if ((e = launch_q40_s16_grouped(a, s)) != hipSuccess) return e;
  } else if ((e = launch_gemv(c.fmt, d, false, s)) != hipSuccess) {
    return e;
  }
  // 6. weighted combine
  const int64_t total = (int64_t)c.m * c.hidden;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, c.out, c.wts,
                     c.y, c.hidden, c.m, c.top_k);
  return hipGetLastError();
}

}  // namespace qg
