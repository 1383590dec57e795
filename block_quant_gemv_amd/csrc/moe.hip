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
//   router_kernel     logits[t, e] = W_r[e] . x[t] (fp32, unquantized x)
//   route_kernel      top-k per token (ties to the lower index), softmax over
//                     the selected logits, then a table that groups the
//                     (token, slot) pairs by expert so each selected expert's
//                     weights are read once for all tokens that chose it
//   grouped GEMV      gate|up of every used expert and of the shared expert,
//                     quantizing x to Q8 blocks in its prologue
//   swiglu_q8         h = silu(g) * u per (token, slot), re-quantized
//   grouped GEMV      down of every used expert and of the shared expert
//   combine_kernel    y[t] = sum_k w[t, k] out[t, k] (slot order) + shared
// Slot rows: token t, slot k (k < top_k routed, k == top_k shared) is row
// t * (top_k + 1) + k of the per-slot intermediates.
#include "common.cuh"
#include "internal.h"
#include "moe.h"
#include "swiglu.h"

namespace qg {

constexpr int kRouterMaxTok = 16;

// One wave per expert row; each lane accumulates float4 chunks of the row
// against the same chunks of every token, then the wave reduces.
__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ wr,
                                                     const float* __restrict__ x,
                                                     float* __restrict__ logits, int n_experts,
                                                     int64_t hidden, int m) {
  const int lane = threadIdx.x & 63;
  const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= n_experts) return;
  const float4* wrow = reinterpret_cast<const float4*>(wr + e * hidden);
  const int64_t nch = hidden / 4;
  float acc[kRouterMaxTok];
#pragma unroll
  for (int t = 0; t < kRouterMaxTok; ++t) acc[t] = 0.0f;
  for (int64_t c = lane; c < nch; c += 64) {
    const float4 w = wrow[c];
#pragma unroll
    for (int t = 0; t < kRouterMaxTok; ++t) {
      if (t < m) {
        const float4 v = reinterpret_cast<const float4*>(x + (int64_t)t * hidden)[c];
        acc[t] = fmaf(w.x, v.x, fmaf(w.y, v.y, fmaf(w.z, v.z, fmaf(w.w, v.w, acc[t]))));
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterMaxTok; ++t) {
    if (t < m) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) logits[(int64_t)t * n_experts + e] = s;
    }
  }
}

// One workgroup of 64 * m threads. Wave t selects token t's top_k experts and
// their softmax weights; then the (token, slot) pairs are grouped by expert
// into the table read by the grouped GEMV (entries of at most kGroupTokens
// tokens, so each expert's weights are read once per 4 tokens that chose it):
//   tbl[0] = number of entries;
//   tbl[1 + e * (2 + kGroupTokens) ...] = {expert, count, slot rows}
// Routed entries come first, ordered by the expert's first occurrence
// (token-major, slot order), tokens ascending; then ceil(m / 4) entries of
// the shared expert (expert = -1) covering every token.
__global__ void route_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                             float* __restrict__ wts, int32_t* __restrict__ tbl, int n_experts,
                             int top_k, int m) {
  extern __shared__ int32_t sh[];
  const int tid = threadIdx.x;
  const int t = tid >> 6, lane = tid & 63;
  const int npairs = m * top_k;
  int32_t* taken = sh;                              // [m * n_experts]
  int32_t* s_ids = taken + m * n_experts;           // [npairs]
  int32_t* first = s_ids + npairs;                  // [npairs] first occurrence index
  int32_t* nchunk = first + npairs;                 // [npairs] chunks of a first occurrence, else 0
  int32_t* rank = nchunk + npairs;                  // [npairs] earlier pairs with the same expert
  int32_t* cnt = rank + npairs;                     // [npairs] total pairs of the expert (first only)

  for (int i = tid; i < m * n_experts; i += blockDim.x) taken[i] = 0;
  __syncthreads();

  if (t < m) {
    const float* lg = logits + (int64_t)t * n_experts;
    int32_t* tk = taken + t * n_experts;
    float my_v = -INFINITY;  // lane k keeps the k-th selection
    int my_i = 0;
    for (int k = 0; k < top_k; ++k) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int e = lane; e < n_experts; e += 64) {
        const float v = lg[e];
        // The first untaken expert always beats the sentinel, so a winner
        // exists even for non-finite logits.
        if (!tk[e] && (bi == 0x7fffffff || v > bv || (v == bv && e < bi))) { bv = v; bi = e; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
      }
      // Every lane now holds the same winner (largest logit, lowest index).
      if (lane == 0) tk[bi] = 1;
      if (lane == k) { my_v = bv; my_i = bi; }
    }
    const float v0 = __shfl(my_v, 0, 64);
    const float ez = (lane < top_k) ? expf(my_v - v0) : 0.0f;
    const float den = wave_sum(ez);
    if (lane < top_k) {
      ids[t * top_k + lane] = my_i;
      wts[t * top_k + lane] = ez / den;
      s_ids[t * top_k + lane] = my_i;
    }
  }
  __syncthreads();

  for (int p = tid; p < npairs; p += blockDim.x) {
    const int e = s_ids[p];
    int f = p, r = 0;
    for (int q = 0; q < p; ++q) {
      if (s_ids[q] == e) {
        if (r == 0) f = q;
        ++r;
      }
    }
    first[p] = f;
    rank[p] = r;
    int c = 0;
    if (f == p)
      for (int q = p; q < npairs; ++q) c += (s_ids[q] == e);
    cnt[p] = c;
    nchunk[p] = (c + kGroupTokens - 1) / kGroupTokens;
  }
  __syncthreads();
  const int tstride = 2 + kGroupTokens;
  for (int p = tid; p < npairs; p += blockDim.x) {
    const int f = first[p];
    int base = 0;
    for (int q = 0; q < f; ++q) base += nchunk[q];
    const int r = rank[p];
    int32_t* ent = tbl + 1 + (int64_t)(base + r / kGroupTokens) * tstride;
    const int tok = p / top_k, k = p - tok * top_k;
    ent[2 + r % kGroupTokens] = tok * (top_k + 1) + k;
    if (r % kGroupTokens == 0) {
      ent[0] = s_ids[p];
      const int left = cnt[f] - r;
      ent[1] = left < kGroupTokens ? left : kGroupTokens;
    }
  }
  if (tid == 0) {
    int routed = 0;
    for (int q = 0; q < npairs; ++q) routed += nchunk[q];
    const int nsh = (m + kGroupTokens - 1) / kGroupTokens;
    for (int c = 0; c < nsh; ++c) {
      int32_t* ent = tbl + 1 + (int64_t)(routed + c) * tstride;
      const int t0 = c * kGroupTokens;
      const int n = (m - t0) < kGroupTokens ? (m - t0) : kGroupTokens;
      ent[0] = -1;
      ent[1] = n;
      for (int j = 0; j < n; ++j) ent[2 + j] = (t0 + j) * (top_k + 1) + top_k;
    }
    tbl[0] = routed + nsh;
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
  // 1. router
  hipLaunchKernelGGL(router_kernel, dim3((unsigned)((c.n_experts + 3) / 4)), dim3(256), 0, s, c.router,
                     c.x, c.logits, c.n_experts, c.hidden, c.m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. top-k, softmax and grouping
  const int npairs = c.m * c.top_k;
  const size_t lds = ((size_t)c.m * c.n_experts + 6 * (size_t)npairs) * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(64 * c.m), lds, s, c.logits, c.ids, c.wts, c.tbl,
                     c.n_experts, c.top_k, c.m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. gate|up of the used experts and the shared expert; the kernel
  // quantizes x in its prologue and the shared-expert workgroup 0 stores the
  // codes in the workspace
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
  g.xf = c.x;
  g.xq_out = c.xq;
  g.dx_out = c.dx;
  g.sx_out = c.sx;
  g.xs = c.hidden;
  g.y = c.gu_out;
  g.ldy = 2 * c.inter;
  g.n = 2 * c.inter;
  g.k = c.hidden;
  g.m = c.m;
  for (int i = 0; i < 4; ++i) g.cb[i] = c.cb[i];
  if ((e = launch_gemv(c.fmt, g, false, s)) != hipSuccess) return e;
  // 4. SwiGLU + re-quantization for every slot row
  if ((e = launch_swiglu_q8(c.gu_out, 2 * c.inter, c.h, c.hq, c.hd, c.hs, (int64_t)c.m * slots, c.inter,
                            s)) != hipSuccess)
    return e;
  // 5. down of the used experts and the shared expert
  GemvProblem d = g;
  d.xf = nullptr;
  d.xq_out = nullptr;
  d.dx_out = nullptr;
  d.sx_out = nullptr;
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
  if ((e = launch_gemv(c.fmt, d, false, s)) != hipSuccess) return e;
  // 6. weighted combine
  const int64_t total = (int64_t)c.m * c.hidden;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, c.out, c.wts,
                     c.y, c.hidden, c.m, c.top_k);
  return hipGetLastError();
}

}  // namespace qg
