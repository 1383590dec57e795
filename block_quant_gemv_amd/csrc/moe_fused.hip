// The MoE expert stage in two launches: routing + gate|up + SwiGLU +
// re-quantization, then down + weighted combine.
//
// The router scores every expert and only the selected experts run; their
// outputs are summed with the softmax weights of the selected logits, plus
// the shared expert ("Understanding Qwen3.6-35B-A3B in llama.cpp", cnblogs,
// section 1.1). Router, top-k, softmax, expert gate/up, SwiGLU, down and the
// weighted sum all stay on the device ("01 · Phase overview: from 2B to 8B
// to MoE", icman.com.cn, stage three); a launch costs several microseconds
// of host and device time, so the stage is merged into as few launches as
// its dependencies allow (the same page's issue ledger, items ㉓ and ㉘:
// merged launches gained more than graph capture alone).
//
// moe_up_kernel: every workgroup first re-derives the routing from the
// router's logits (at most 16 tokens x 1024 experts of fp32 in L2): top-k per
// token by repeated wave-wide maxima of an order-preserving (logit, expert)
// key, softmax over the selected logits, then the table of entries: first
// the shared expert's (its tokens in groups of four, so that its items weigh
// about as much as a routed expert's and are taken first), then one per
// distinct selected expert, in order of first selection (token-major, slot
// order), holding every token that chose it. All workgroups build the same
// table, so no grid-wide hand-off is needed, and each distinct expert's
// weights are read once for all of its tokens. An item is (entry, 32
// consecutive elements of h): the 32 gate rows and the 32 matching up rows
// of the expert, so the workgroup holds both halves of SwiGLU and a whole Q8
// block of h, which it re-quantizes itself (32 lanes per token). Sixteen
// waves take four rows each, loaded as one coalesced range into the wave's
// LDS tile and decoded with the format views the decode GEMV uses, one row
// per 16-lane group (so one 16-lane reduction serves all four rows); the
// activations (the router launch's Q8 codes of x) are staged in LDS once.
//
// moe_down_kernel: an item is (token, block of output rows). Wave s takes
// slot s (routed slots in order, then the shared expert): its expert's rows
// of the block as one coalesced range, the slot's re-quantized h in
// registers. The slots' row sums meet in LDS and are combined in slot order
// (weight times routed output, then plus the shared output), so the result
// is bitwise reproducible without atomics.
#include "common.cuh"
#include "formats.cuh"
#include "internal.h"
#include "moe.h"
#include "route.cuh"
#include "s16.cuh"

#include <type_traits>

namespace qg {

namespace {

constexpr int kUpWaves = 16;        // waves per moe_up_kernel workgroup
constexpr int kUpRows = 4;          // rows per wave per item (16 waves x 4 = 64 = 32 gate + 32 up)
// LDS bytes between the rows of a wave's up tile. The four rows are read
// together (one per 16-lane group); their natural pitch of 1152 B is a
// multiple of the bank period, so the groups hit the same banks. 32 B apart
// (measured on MI355X, Q4_0 hidden 2048: 16 tokens 58.8 -> 57.0 us per layer,
// 4 tokens 28.3 -> 27.5 us; 16 B gained less, 64 B no more).
constexpr int kPad = 32;
constexpr int kUpTok = 2;         // tokens per accumulation pass
constexpr int kUpLPL = 9;           // 16-byte loads per lane: a wave's four rows, at most 9216 B
constexpr int kDnLPL = 5;           // 16-byte loads per lane in moe_down_kernel
constexpr int kMaxTok = 16;         // tokens a launch can hold
// Tokens up to which the two-launch expert stage is used. Measured on MI355X
// (256 experts, top-8 + shared, hidden 2048, expert intermediate 512, Q4_0,
// expert weights from HBM): 16.5 / 23.7 / 30.6 / 43.1 / 70.3 us at 1 / 2 / 4
// / 8 / 16 tokens against 24.4 / 29.2 / 37.7 / 48.9 / 75.0 us for the
// six-launch path, once the shared expert's tokens are split over entries of
// kShareTok tokens that are taken first (one entry with all 16 tokens, last:
// 100 us at 16 tokens).
constexpr int kFusedMaxTok = kMaxTok;
constexpr int kMaxPairs = kMaxTok * 16;
// moe_up_kernel's gate|up sums of an item, [token][64], two of them: items
// alternate, so SwiGLU of one item and the decode of the next can overlap.
constexpr int kUpSgu = 2 * kMaxTok * 64 * 4;
// Tokens per shared-expert entry: the shared expert serves every token, so
// its tokens are split over several entries (each reads the shared weights
// again, mostly from cache) to keep its items as light as the routed ones.
constexpr int kShareTok = 4;
// LDS bytes per token of staged 16-bit activation codes: the 16 dwords of
// paired codes of each 32-element unit as four 16-byte quarters, quarter v
// of unit u at 16 (v U + u) (lanes reading consecutive units read
// consecutive words: no LDS bank conflicts), then per unit (scale, code sum).
__host__ __device__ constexpr int act16_token_bytes(int U) { return 72 * U; }
constexpr int kMaxShare = (kMaxTok + kShareTok - 1) / kShareTok;
constexpr int kBufDword3 = 0x00020000;
constexpr int kNonTemporal = 2;

// Routing of one call, identical in every workgroup (LDS).
constexpr int kMaxExperts = 1024;

struct alignas(16) Route {
  int32_t ids[kMaxPairs];       // [token][slot] selected expert
  float wts[kMaxPairs];         // [token][slot] softmax weight
  int32_t ent_expert[kMaxPairs + kMaxShare];
  uint32_t ent_mask[kMaxPairs + kMaxShare];  // tokens of the entry, bit t
  uint32_t tok_mask[kMaxExperts];    // per expert: tokens that chose it
  int32_t first_pair[kMaxExperts];   // per expert: its first (token, slot) pair
  int32_t wave_first[kMaxPairs / 64];
  int32_t n_entries;
};

// Wave `wid` < m selects token wid's top_k experts (ties to the lower index)
// and their softmax weights; then the entries are built. Ends with a barrier.
// NPL: logits per lane (n_experts <= 64 * NPL).
template <int NPL>
QG_DEV void build_route(Route& R, const float* __restrict__ logits, int n_experts, int top_k, int m, int wid,
                        int lane, int nthreads) {
  const int tid = threadIdx.x;
  if (wid < m) {
    const float* lg = logits + (int64_t)wid * n_experts;
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < n_experts ? lg[e] : 0.0f;
    }
    uint32_t taken = 0;  // bit i: expert lane + 64 i selected (or absent)
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i >= n_experts) taken |= 1u << i;
    float my_v = -INFINITY;  // lane k keeps the k-th selection
    int my_i = 0;
    for (int k = 0; k < top_k; ++k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const uint64_t key = route_key(v[i], lane + 64 * i);
        if (!((taken >> i) & 1u) && key > best) best = key;
      }
      best = wave_max_key(best);
      const int bi = route_key_expert(best);
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == k) {
        my_v = route_key_value(best);
        my_i = bi;
      }
    }
    const float v0 = __shfl(my_v, 0, 64);
    const float ez = (lane < top_k) ? expf(my_v - v0) : 0.0f;
    const float den = wave_sum(ez);
    if (lane < top_k) {
      R.ids[wid * top_k + lane] = my_i;
      R.wts[wid * top_k + lane] = ez / den;
    }
  }
  for (int i = tid; i < n_experts; i += nthreads) {
    R.tok_mask[i] = 0u;
    R.first_pair[i] = 0x7fffffff;
  }
  __syncthreads();
  // Pair p (token p / top_k, slot p % top_k) opens an entry when no earlier
  // pair chose the same expert; the entry holds every token that chose it.
  const int np = m * top_k;
  if (tid < np) {
    const int ex = R.ids[tid];
    atomicOr(&R.tok_mask[ex], 1u << (tid / top_k));
    atomicMin(&R.first_pair[ex], tid);
  }
  __syncthreads();
  bool first = false;
  uint32_t mask = 0;
  int e = -1;
  if (tid < np) {
    e = R.ids[tid];
    first = R.first_pair[e] == tid;
    mask = R.tok_mask[e];
  }
  // Entry index = number of first pairs before this one (np <= 256: at most
  // four waves of pairs).
  const uint64_t bal = __ballot(first);
  if (lane == 0 && wid < kMaxPairs / 64) R.wave_first[wid] = __popcll(bal);
  __syncthreads();
  // The shared expert's entries come first (kShareTok tokens each), so
  // their heavier items are taken at the start rather than at the tail.
  const int nsh = (m + kShareTok - 1) / kShareTok;
  if (first) {
    int idx = __popcll(bal & ((1ull << lane) - 1ull));
    for (int w = 0; w < wid; ++w) idx += R.wave_first[w];
    R.ent_expert[nsh + idx] = e;
    R.ent_mask[nsh + idx] = mask;
  }
  if (tid < nsh) {
    const int t0 = kShareTok * tid, t1 = (t0 + kShareTok) < m ? (t0 + kShareTok) : m;
    R.ent_expert[tid] = -1;
    R.ent_mask[tid] = (uint32_t)((1ull << t1) - (1ull << t0));
  }
  if (tid == 0) {
    int nr = 0;
    for (int w = 0; w < (np + 63) / 64; ++w) nr += R.wave_first[w];
    R.n_entries = nr + nsh;
  }
  __syncthreads();
}

// Slot of expert e in token t's selection (the shared expert: top_k).
QG_DEV int slot_of(const Route& R, int t, int e, int top_k) {
  if (e < 0) return top_k;
  int s = 0;
  for (int k = 0; k < top_k; ++k)
    if (R.ids[t * top_k + k] == e) s = k;
  return s;
}

// A staged unit of 16-bit codes (see act16_token_bytes): LDS reads only.
QG_DEV Act16 load_act16(const uint8_t* tok, int U, int u) {
  Act16 x;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(tok + 16 * (v * U + u));
    x.p[4 * v + 0] = q.x;
    x.p[4 * v + 1] = q.y;
    x.p[4 * v + 2] = q.z;
    x.p[4 * v + 3] = q.w;
  }
  const int2 ms = *reinterpret_cast<const int2*>(tok + 64 * U + 8 * u);
  x.dx = __int_as_float(ms.x);
  x.sum = ms.y;
  return x;
}

}  // namespace

struct MoeFusedArgs {
  const float* logits;
  int n_experts, top_k, m;
  int32_t* ids_out;
  float* wts_out;
  const uint8_t *gu, *gu_shared, *dn, *dn_shared;
  int64_t gu_stride, dn_stride;
  const int8_t* xq;
  const int16_t* xq16;      // 16-bit codes of x instead of xq (S16 kernels)
  const float* dx;
  const int32_t* sx;        // code sums of the 16-bit blocks of x
  int64_t hidden, inter;
  int64_t rb_gu, rb_dn;     // row bytes of gate|up (K = hidden) and down (K = inter)
  float* gu_out;            // [m * (top_k + 1), 2 inter]
  float* h_out;             // [m * (top_k + 1), inter]
  int8_t* hq;
  int16_t* hq16;            // 16-bit codes of h instead of hq (S16 kernels)
  float* hd;
  int32_t* hs;
  float* y;                 // [m, hidden]
  uint32_t cb[4];
  int act_bytes;            // LDS bytes of the staged activations (m tokens)
  int tile_bytes;           // LDS bytes of one wave's weight tile
  int dn_rows;              // output rows per down item
};

// ------------------------------------------------------------ gate|up --

// LPL: 16-byte loads per lane (a wave's four rows); NPL: logits per lane in
// the routing prologue (n_experts <= 64 NPL); S16: 16-bit activation codes
// of x and h (Q4_0 experts) instead of Q8 codes.
template <int FMT, int LPL, int NPL, bool S16>
__global__ __launch_bounds__(kUpWaves * 64) void moe_up_kernel(const MoeFusedArgs a) {
  using F = typename FmtOf<FMT>::T;
  static_assert(!S16 || FMT == kQ4_0, "16-bit activations are for Q4_0 experts");
  extern __shared__ __align__(16) uint8_t smem[];
  Route& R = *reinterpret_cast<Route*>(smem);
  float* s_gu2 = reinterpret_cast<float*>(smem + sizeof(Route));  // [2][kMaxTok][64]
  uint8_t* act = smem + sizeof(Route) + kUpSgu;                     // staged activations
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  uint8_t* tile = act + a.act_bytes + wid * a.tile_bytes;

  const int U = (int)(a.hidden / 32);      // 32-element units per row (multiple of 64)
  const int tokb = S16 ? act16_token_bytes(U) : act_token_bytes(U);
  // Activations of every token (the router launch's Q8 or 16-bit codes of
  // x), staged once per workgroup: token t at act + t * tokb. The loads are
  // issued before the routing's logit loads so both round trips overlap.
  constexpr int kStage = 2;  // (token, unit) tasks per thread: m * U <= 2048
  constexpr int kStW = S16 ? 16 : 8;  // dwords of codes per unit
  uint32_t st_c[kStage][kStW];
  float st_d[kStage];
  int st_s[kStage];
#pragma unroll
  for (int r = 0; r < kStage; ++r) {
    const int i = threadIdx.x + r * kUpWaves * 64;
    if (i < a.m * U) {
      const int t = i / U, u = i - t * U;
      const int4* xr = S16 ? reinterpret_cast<const int4*>(a.xq16 + (int64_t)t * a.hidden + 32 * u)
                           : reinterpret_cast<const int4*>(a.xq + (int64_t)t * a.hidden + 32 * u);
#pragma unroll
      for (int v = 0; v < kStW / 4; ++v) {
        const int4 q = xr[v];
        st_c[r][4 * v + 0] = (uint32_t)q.x;
        st_c[r][4 * v + 1] = (uint32_t)q.y;
        st_c[r][4 * v + 2] = (uint32_t)q.z;
        st_c[r][4 * v + 3] = (uint32_t)q.w;
      }
      st_d[r] = a.dx[(int64_t)t * U + u];
      if constexpr (S16) st_s[r] = a.sx[(int64_t)t * U + u];
    }
  }
  build_route<NPL>(R, a.logits, a.n_experts, a.top_k, a.m, wid, lane, blockDim.x);
#pragma unroll
  for (int r = 0; r < kStage; ++r) {
    const int i = threadIdx.x + r * kUpWaves * 64;
    if (i < a.m * U) {
      const int t = i / U, u = i - t * U;
      uint8_t* tok = act + t * tokb;
      if constexpr (S16) {
        // paired codes of the unit, then (scale, code sum)
        uint32_t pr[16];
        pair16(st_c[r], pr);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<u32x4*>(tok + 16 * (v * U + u)) = u32x4{pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]};
        *reinterpret_cast<int2*>(tok + 64 * U + 8 * u) = make_int2(__float_as_int(st_d[r]), st_s[r]);
      } else {
        const int ones = 0x01010101;
        const int4 lo = make_int4((int)st_c[r][0], (int)st_c[r][1], (int)st_c[r][2], (int)st_c[r][3]);
        const int4 hi = make_int4((int)st_c[r][4], (int)st_c[r][5], (int)st_c[r][6], (int)st_c[r][7]);
        const int sa = dot4(lo.x, ones, dot4(lo.y, ones, dot4(lo.z, ones, dot4(lo.w, ones, 0))));
        const int sb = dot4(hi.x, ones, dot4(hi.y, ones, dot4(hi.z, ones, dot4(hi.w, ones, 0))));
        *reinterpret_cast<int4*>(tok + 16 * u) = lo;
        *reinterpret_cast<int4*>(tok + 16 * U + 16 * u) = hi;
        *reinterpret_cast<int2*>(tok + 32 * U + 8 * u) = make_int2(__float_as_int(st_d[r]), (sa & 0xffff) | (sb << 16));
      }
    }
  }
  __syncthreads();
  const int np = a.m * a.top_k;
  if (blockIdx.x == 0)
    for (int p = threadIdx.x; p < np; p += blockDim.x) {
      a.ids_out[p] = R.ids[p];
      a.wts_out[p] = R.wts[p];
    }

  const int tiles = (int)(a.inter / 32);
  const int n_items = R.n_entries * tiles;
  const int S1 = a.top_k + 1;
  uint32_t cbr[4] = {a.cb[0], a.cb[1], a.cb[2], a.cb[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(cbr[i]));

  // The byte range of this wave's four rows of an item: virtual rows
  // 4 wid .. 4 wid + 3 (0..31 gate, 32..63 up), contiguous in the matrix.
  const int v0 = kUpRows * wid;
  const int rr = lane >> 4, lam = lane & 15;
  const int cpr = (int)(a.rb_gu / 16);  // this lane's row of the four, and unit phase
  auto item_range = [&](int item, const uint8_t*& W, int64_t& b0) __attribute__((always_inline)) {
    const int en = item / tiles, j = item - en * tiles;
    const int e = R.ent_expert[en];
    W = e < 0 ? a.gu_shared : a.gu + (int64_t)e * a.gu_stride;
    const int64_t row0 = v0 < 32 ? (int64_t)32 * j + v0 : a.inter + (int64_t)32 * j + (v0 - 32);
    b0 = row0 * a.rb_gu;
  };
  // Loads of an item's rows (items past the end read zeros from an empty
  // range, with no memory access): issued one item ahead, after the
  // previous item's decode, so they are in flight during its SwiGLU and the
  // next item's start.
  auto issue = [&](u32x4 (&buf)[LPL], int item) __attribute__((always_inline)) {
    const uint8_t* W = a.gu_shared;
    int64_t b0 = 0;
    int nch = 0;
    if (item < n_items) {
      item_range(item, W, b0);
      nch = (int)(((b0 + kUpRows * a.rb_gu + 15) & ~(int64_t)15) - (b0 & ~(int64_t)15)) >> 4;
    }
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W + (b0 & ~(int64_t)15)), 0, nch * 16, kBufDword3);
#pragma unroll
    for (int i = 0; i < LPL; ++i)
      buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + 64 * i) * 16, 0, kNonTemporal);
  };
  u32x4 buf[LPL];
  issue(buf, blockIdx.x);

  int half = 0;  // which half of s_gu2 this item uses
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    float* s_gu = s_gu2 + half * (kMaxTok * 64);
    half ^= 1;
    const int en = item / tiles, j = item - en * tiles;
    const int e = R.ent_expert[en];
    const uint32_t mask = R.ent_mask[en];
    const int c = __popc(mask);
    const uint8_t* W;
    int64_t b0;
    item_range(item, W, b0);
    const int64_t a0 = b0 & ~(int64_t)15;
    const int nch = (int)(((b0 + kUpRows * a.rb_gu + 15) & ~(int64_t)15) - a0) >> 4;

    // Weights to the wave's LDS tile, then decode.
#pragma unroll
    for (int i = 0; i < LPL; ++i) {
      const int ch = lane + 64 * i;
      // rows start on 16-byte chunks (row bytes are a multiple of 16):
      // chunk ch belongs to row ch / cpr
      if (ch < nch) *reinterpret_cast<u32x4*>(tile + 16 * ch + (ch / cpr) * kPad) = buf[i];
    }
    // Each 16-lane row of the wave takes one of its four rows (lane l:
    // row l / 16, units l % 16 + 16 i), so a row's sum is a 16-lane
    // reduction and one reduction serves all four rows.
    const uint32_t base = (uint32_t)(b0 - a0) + (uint32_t)(rr * (a.rb_gu + kPad));
    // Tokens in chunks of kUpTok (accumulators stay in registers); the
    // weights are decoded from LDS again for each chunk.
    uint32_t mrem = mask;  // tokens of the entry not yet taken, ascending
    for (int t0 = 0; t0 < c; t0 += kUpTok) {
      int tok[kUpTok];  // token ids of this chunk
#pragma unroll
      for (int t = 0; t < kUpTok; ++t) {
        tok[t] = mrem ? __builtin_ctz(mrem) : 0;
        mrem &= mrem - 1;
      }
      float acc[kUpTok];
#pragma unroll
      for (int t = 0; t < kUpTok; ++t) acc[t] = 0.0f;
      for (int u = lam; u < U; u += 16) {
        const uint32_t uoff = (uint32_t)((u / F::kUPB) * F::kBB);
        const int sub = u % F::kUPB;
        const typename F::W w = F::load(tile, base + uoff, sub, cbr);
#pragma unroll
        for (int t = 0; t < kUpTok; ++t) {
          if (t0 + t < c) {
            if constexpr (S16) {
              const Act16 x = load_act16(act + tok[t] * tokb, U, u);
              acc[t] = fmaf((float)(q4_dot16(w.q, x.p) - 8 * x.sum), x.dx * w.d, acc[t]);
            } else {
              acc[t] = F::fma(w, load_act(act + tok[t] * tokb, U, u), acc[t]);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kUpTok; ++t) {
        if (t0 + t < c) {
          const float sum = group_sum16(acc[t], 16);
          if (lam == 0) s_gu[(t0 + t) * 64 + v0 + rr] = sum;
        }
      }
    }
    // The next item's rows are requested only now, after this item's
    // decode: requested before it (more bytes in flight per CU), the layer
    // measured slower on MI355X (16 tokens 56.7 against 55.6 us; requested
    // after the SwiGLU, 60.5 us).
    issue(buf, item + gridDim.x);
    __syncthreads();

    // SwiGLU and Q8 re-quantization of the item's 32 elements of h, 32
    // lanes per token, one element each (the activation quantizer's
    // arithmetic: the block's absolute maximum, d = amax / 127, the codes
    // and their sum).
    if ((int)threadIdx.x < 32 * c) {
      const int i = threadIdx.x >> 5, el = threadIdx.x & 31;
      int t = -1;
      for (int q = 0; q <= i; ++q) t = __builtin_ffs(mask >> (t + 1)) + t;
      const int64_t row = (int64_t)t * S1 + slot_of(R, t, e, a.top_k);
      const float g = s_gu[i * 64 + el];
      const float up = s_gu[i * 64 + 32 + el];
      const float h = g / (1.0f + expf(-g)) * up;
      const int64_t col = (int64_t)32 * j + el;
      a.gu_out[row * 2 * a.inter + col] = g;
      a.gu_out[row * 2 * a.inter + a.inter + col] = up;
      a.h_out[row * a.inter + col] = h;
      float amax = max8(fabsf(h));
      amax = fmaxf(amax, dpp<0x140>(amax));           // 16 lanes (row_mirror)
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));  // 32 lanes
      const float d = (amax > 0.0f) ? amax / (S16 ? 32767.0f : 127.0f) : 0.0f;
      int q;
      if constexpr (S16) {
        q = d != 0.0f ? code16(h, d) : 0;
        a.hq16[row * a.inter + col] = (int16_t)q;
      } else {
        q = d != 0.0f ? q8_code(h, d, __builtin_amdgcn_rcpf(d)) : 0;
        a.hq[row * a.inter + col] = (int8_t)q;
      }
      int qs = sum4(q);
      qs += other_quad(qs);
      qs += dpp_i<0x140>(qs);        // 16 lanes
      qs += __shfl_xor(qs, 16, 64);  // 32 lanes
      if (el == 0) {
        a.hd[row * (a.inter / 32) + j] = d;
        a.hs[row * (a.inter / 32) + j] = qs;
      }
    }
    // No barrier here: the next item writes the other half of s_gu2, and
    // its own barrier (after its decode) orders these reads before the
    // item after it writes this half again. The waves that do no SwiGLU
    // go on to the next item's decode at once.
  }
}

// ---------------------------------------------------------- down + combine --

// LPR: lanes per row (units of h per row, <= 64); JU: units per lane; S16:
// 16-bit codes of h (Q4_0 experts).
template <int FMT, int LPR, int JU, bool S16>
__global__ __launch_bounds__(1024) void moe_down_kernel(const MoeFusedArgs a) {
  using F = typename FmtOf<FMT>::T;
  static_assert(!S16 || FMT == kQ4_0, "16-bit activations are for Q4_0 experts");
  extern __shared__ __align__(16) uint8_t smem[];
  const int S1 = a.top_k + 1;
  const int RB = a.dn_rows;                         // output rows per item (multiple of 64 / LPR)
  float* s_out = reinterpret_cast<float*>(smem);   // [S1][RB]
  int32_t* s_ids = reinterpret_cast<int32_t*>(smem + kMaxTok * 64 * 4);  // [m][top_k]
  float* s_wts = reinterpret_cast<float*>(s_ids + kMaxPairs);             // [m][top_k]
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's slot
  const int lane = threadIdx.x & 63;
  uint8_t* tile = smem + (size_t)kMaxTok * 64 * sizeof(float) + 2 * kMaxPairs * 4 + s * a.tile_bytes;
  constexpr int RPP = 64 / LPR;
  const int lam = lane % LPR, rho = lane / LPR;
  const int U = (int)(a.inter / 32);
  const int nblk = (int)((a.hidden + RB - 1) / RB);
  const int n_items = a.m * nblk;
  uint32_t cbr[4] = {a.cb[0], a.cb[1], a.cb[2], a.cb[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(cbr[i]));
  // The routing (expert ids and weights of every pair) to LDS once: items
  // then find their experts and combine weights without global-memory
  // round trips (measured: 8 tokens 40.7 -> 39.3 us per layer). Requesting
  // the next item's h ahead with its weights measured slower (47 us at 8
  // tokens) and is not done.
  for (int p = threadIdx.x; p < a.m * a.top_k; p += blockDim.x) {
    s_ids[p] = a.ids_out[p];
    s_wts[p] = a.wts_out[p];
  }
  __syncthreads();

  // The byte range of this wave's slot's rows of an item.
  auto item_range = [&](int item, const uint8_t*& W, int64_t& b0, int& nrows) __attribute__((always_inline)) {
    const int t = item / nblk, blk = item - t * nblk;
    const int64_t r0 = (int64_t)blk * RB;
    nrows = (int)((a.hidden - r0) < RB ? (a.hidden - r0) : RB);
    const int e = s < a.top_k ? s_ids[t * a.top_k + s] : -1;
    W = e < 0 ? a.dn_shared : a.dn + (int64_t)e * a.dn_stride;
    b0 = r0 * a.rb_dn;
  };
  // Loads of an item's rows, issued one item ahead, after the current
  // item's decode (items past the end read
  // zeros from an empty range, with no memory access).
  auto issue = [&](u32x4 (&buf)[kDnLPL], int item) __attribute__((always_inline)) {
    const uint8_t* W = a.dn_shared;
    int64_t b0 = 0;
    int nrows = 0, nch = 0;
    if (item < n_items) {
      item_range(item, W, b0, nrows);
      nch = (int)(((b0 + nrows * a.rb_dn + 15) & ~(int64_t)15) - (b0 & ~(int64_t)15)) >> 4;
    }
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W + (b0 & ~(int64_t)15)), 0, nch * 16, kBufDword3);
#pragma unroll
    for (int i = 0; i < kDnLPL; ++i)
      buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + 64 * i) * 16, 0, kNonTemporal);
  };
  u32x4 buf[kDnLPL];
  issue(buf, blockIdx.x);

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int t = item / nblk, blk = item - t * nblk;
    const int64_t r0 = (int64_t)blk * RB;
    const uint8_t* W;
    int64_t b0;
    int nrows;
    item_range(item, W, b0, nrows);
    const int64_t a0 = b0 & ~(int64_t)15;
    const int nch = (int)(((b0 + nrows * a.rb_dn + 15) & ~(int64_t)15) - a0) >> 4;
    // The slot's re-quantized h (requested before the next item's weights,
    // so waiting for it never waits for them): this lane's units lam + LPR jj.
    const int64_t hrow = (int64_t)t * S1 + s;
    std::conditional_t<S16, Act16, Act> x[JU];
#pragma unroll
    for (int jj = 0; jj < JU; ++jj) {
      const int u = lam + LPR * jj;
      if constexpr (S16) {
        const int4* hp = reinterpret_cast<const int4*>(a.hq16 + hrow * a.inter + 32 * u);
        uint32_t w16[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int4 q = hp[v];
          w16[4 * v + 0] = (uint32_t)q.x;
          w16[4 * v + 1] = (uint32_t)q.y;
          w16[4 * v + 2] = (uint32_t)q.z;
          w16[4 * v + 3] = (uint32_t)q.w;
        }
        pair16(w16, x[jj].p);
        x[jj].sum = a.hs[hrow * U + u];
      } else {
        const int4 lo = reinterpret_cast<const int4*>(a.hq + hrow * a.inter)[2 * u];
        const int4 hi = reinterpret_cast<const int4*>(a.hq + hrow * a.inter)[2 * u + 1];
        x[jj].x[0] = lo.x; x[jj].x[1] = lo.y; x[jj].x[2] = lo.z; x[jj].x[3] = lo.w;
        x[jj].x[4] = hi.x; x[jj].x[5] = hi.y; x[jj].x[6] = hi.z; x[jj].x[7] = hi.w;
      }
      x[jj].dx = a.hd[hrow * U + u];
    }
#pragma unroll
    for (int i = 0; i < kDnLPL; ++i) {
      const int ch = lane + 64 * i;
      if (ch < nch) *reinterpret_cast<u32x4*>(tile + 16 * ch) = buf[i];
    }
    if constexpr (!S16) {
#pragma unroll
      for (int jj = 0; jj < JU; ++jj) {
        const int ones = 0x01010101;
        x[jj].sa = dot4(x[jj].x[0], ones, dot4(x[jj].x[1], ones, dot4(x[jj].x[2], ones, dot4(x[jj].x[3], ones, 0))));
        x[jj].sb = dot4(x[jj].x[4], ones, dot4(x[jj].x[5], ones, dot4(x[jj].x[6], ones, dot4(x[jj].x[7], ones, 0))));
      }
    }
    const uint32_t base = (uint32_t)(b0 - a0);
    for (int p = 0; p * RPP < nrows; ++p) {
      int rl = p * RPP + rho;
      const bool valid = rl < nrows;
      rl = valid ? rl : nrows - 1;
      float acc = 0.0f;
#pragma unroll
      for (int jj = 0; jj < JU; ++jj) {
        const int u = lam + LPR * jj;
        const typename F::W w =
            F::load(tile, base + (uint32_t)(rl * a.rb_dn) + (uint32_t)((u / F::kUPB) * F::kBB), u % F::kUPB, cbr);
        if constexpr (S16)
          acc = fmaf((float)(q4_dot16(w.q, x[jj].p) - 8 * x[jj].sum), x[jj].dx * w.d, acc);
        else
          acc = F::fma(w, x[jj], acc);
      }
      const float sum = group_sum(acc, LPR);
      if (lam == 0 && valid) s_out[s * RB + rl] = sum;
    }
    // The next item's rows, requested after this item's decode (as in the
    // gate|up kernel: 16 tokens 55.5 -> 54.9 us).
    issue(buf, item + gridDim.x);
    __syncthreads();
    // y = sum over routed slots in order of weight * output, plus the shared expert.
    for (int r = threadIdx.x; r < nrows; r += blockDim.x) {
      float acc = 0.0f;
      for (int k = 0; k < a.top_k; ++k) acc = fmaf(s_wts[t * a.top_k + k], s_out[k * RB + r], acc);
      a.y[(int64_t)t * a.hidden + r0 + r] = acc + s_out[a.top_k * RB + r];
    }
    __syncthreads();  // s_out and the tiles are reused by the next item
  }
}

// ------------------------------------------------------------- launchers --

namespace {

size_t up_lds(const MoeFusedArgs& a) {
  return sizeof(Route) + (size_t)kUpSgu + (size_t)a.act_bytes +
         (size_t)kUpWaves * a.tile_bytes;
}

template <int FMT, int LPL, int NPL, bool S16>
hipError_t launch_up_t(const MoeFusedArgs& a, int n_items_max, hipStream_t s) {
  auto kern = moe_up_kernel<FMT, LPL, NPL, S16>;
  const size_t lds = up_lds(a);
  int per_cu = 0, cus = 0;
  hipError_t e = kernel_residency(reinterpret_cast<const void*>(kern), kUpWaves * 64, lds, true, &per_cu, &cus);
  if (e != hipSuccess) return e;
  int64_t grid = (int64_t)cus * per_cu;
  if (grid > n_items_max) grid = n_items_max;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kUpWaves * 64), lds, s, a);
  return hipGetLastError();
}

// Loads per lane for a wave's four rows of rb bytes (plus alignment).
int up_loads(int64_t rb) { return (int)((kUpRows * rb + 32 + 1023) / 1024); }

template <int FMT, bool S16 = false>
hipError_t launch_up_npl(const MoeFusedArgs& a, int n_items_max, hipStream_t s) {
  const bool small = up_loads(a.rb_gu) <= 5;
  if (a.n_experts <= 256)
    return small ? launch_up_t<FMT, 5, 4, S16>(a, n_items_max, s)
                 : launch_up_t<FMT, kUpLPL, 4, S16>(a, n_items_max, s);
  return small ? launch_up_t<FMT, 5, 16, S16>(a, n_items_max, s)
               : launch_up_t<FMT, kUpLPL, 16, S16>(a, n_items_max, s);
}

// Output rows per down item: a.dn_rows or twice that when a wave's rows
// still fit its loads. An item costs about as much as kDnItemRows rows more
// than its rows, and the workgroups take the items in rounds, so the choice
// with fewer rounds x (rows + kDnItemRows) wins (measured on MI355X, Q4_0,
// hidden 2048, expert intermediate 512: 16 rows at 16 tokens 70.4 -> 66.7 us
// per layer; 8 rows stay best where a round more would be needed).
constexpr int kDnItemRows = 8;

template <int FMT, int LPR, int JU, bool S16 = false>
hipError_t launch_dn_t(MoeFusedArgs a, hipStream_t s) {
  auto kern = moe_down_kernel<FMT, LPR, JU, S16>;
  const int S1 = a.top_k + 1;
  const int rows0 = a.dn_rows;
  int64_t best_cost = -1, best_grid = 0;
  size_t best_lds = 0;
  for (int rows = rows0; rows <= 2 * rows0; rows *= 2) {
    if (rows > rows0 && rows * a.rb_dn + 32 > (int64_t)kDnLPL * 1024) break;
    const int tile = (int)((rows * a.rb_dn + 32 + 15) / 16 * 16 + 16);
    const size_t lds = (size_t)kMaxTok * 64 * sizeof(float) + 2 * kMaxPairs * 4 + (size_t)S1 * tile;
    int per_cu = 0, cus = 0;
    hipError_t e = kernel_residency(reinterpret_cast<const void*>(kern), S1 * 64, lds, true, &per_cu, &cus);
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)a.m * ((a.hidden + rows - 1) / rows);
    int64_t grid = (int64_t)cus * per_cu;
    if (grid > items) grid = items;
    if (grid < 1) grid = 1;
    const int64_t cost = (items + grid - 1) / grid * (rows + kDnItemRows);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_grid = grid;
      best_lds = lds;
      a.dn_rows = rows;
      a.tile_bytes = tile;
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)best_grid), dim3(S1 * 64), best_lds, s, a);
  return hipGetLastError();
}

}  // namespace

bool moe_fused_ok(const MoeCall& c) {
  const int64_t rb_gu = fmt_row_bytes(c.fmt, c.hidden), rb_dn = fmt_row_bytes(c.fmt, c.inter);
  if (rb_gu <= 0 || rb_dn <= 0) return false;
  const int64_t U = c.inter / 32;
  if (c.m < 1 || c.m > kFusedMaxTok || c.top_k < 1 || c.top_k > 15 || c.n_experts > kMaxExperts) return false;
  const bool s16 = c.xq16 != nullptr;
  if (s16 && (c.fmt != kQ4_0 || !c.hq16 || !c.sx || !c.hs)) return false;
  if (c.hidden % 2048 || c.hidden > 8192 || c.inter % 32 || c.m * (c.hidden / 32) > 2048) return false;
  if (U != 16 && U != 32 && U != 64 && U != 128) return false;
  if (up_loads(rb_gu) > kUpLPL || rb_gu % 16) return false;   // a wave's four rows in one load
  const int rpp = 64 / (int)(U < 64 ? U : 64);
  const int rows = rpp * 2 > 8 ? rpp * 2 : 8;
  if (rows * rb_dn + 32 > (int64_t)kDnLPL * 1024) return false;
  const int tokb = s16 ? act16_token_bytes((int)(c.hidden / 32)) : act_token_bytes((int)(c.hidden / 32));
  const size_t up = sizeof(Route) + (size_t)kUpSgu + (size_t)c.m * tokb +
                    (size_t)kUpWaves * (size_t)((kUpRows * (rb_gu + kPad) + 32 + 15) / 16 * 16 + 16);
  return up <= (size_t)kLdsBytes;
}

hipError_t launch_moe_fused(const MoeCall& c, hipStream_t s) {
  if (!moe_fused_ok(c)) return hipErrorInvalidValue;
  MoeFusedArgs a;
  a.logits = c.logits;
  a.n_experts = c.n_experts;
  a.top_k = c.top_k;
  a.m = c.m;
  a.ids_out = c.ids;
  a.wts_out = c.wts;
  a.gu = c.gu;
  a.gu_shared = c.gu_shared;
  a.dn = c.dn;
  a.dn_shared = c.dn_shared;
  a.gu_stride = c.gu_stride;
  a.dn_stride = c.dn_stride;
  a.xq = c.xq;
  a.xq16 = c.xq16;
  a.dx = c.dx;
  a.sx = c.sx;
  a.hidden = c.hidden;
  a.inter = c.inter;
  a.rb_gu = fmt_row_bytes(c.fmt, c.hidden);
  a.rb_dn = fmt_row_bytes(c.fmt, c.inter);
  a.gu_out = c.gu_out;
  a.h_out = c.h;
  a.hq = c.hq;
  a.hq16 = c.hq16;
  a.hd = c.hd;
  a.hs = c.hs;
  a.y = c.y;
  for (int i = 0; i < 4; ++i) a.cb[i] = c.cb[i];
  const bool s16 = c.xq16 != nullptr;  // Q4_0 experts (moe_fused_ok)
  a.act_bytes = c.m * (s16 ? act16_token_bytes((int)(c.hidden / 32)) : act_token_bytes((int)(c.hidden / 32)));
  a.tile_bytes = (int)((kUpRows * (a.rb_gu + kPad) + 32 + 15) / 16 * 16 + 16);
  const int U = (int)(c.inter / 32);
  const int rpp = 64 / (U < 64 ? U : 64);
  a.dn_rows = rpp * 2 > 8 ? rpp * 2 : 8;
  // Entries: at most one per (token, slot) pair, plus the shared expert's.
  const int n_items_max = (c.m * c.top_k + (c.m + kShareTok - 1) / kShareTok) * (int)(c.inter / 32);
  hipError_t e;
  if (s16) {
    if ((e = launch_up_npl<kQ4_0, true>(a, n_items_max, s)) != hipSuccess) return e;
    switch (U) {
      case 16: return launch_dn_t<kQ4_0, 16, 1, true>(a, s);
      case 32: return launch_dn_t<kQ4_0, 32, 1, true>(a, s);
      case 64: return launch_dn_t<kQ4_0, 64, 1, true>(a, s);
      default: return launch_dn_t<kQ4_0, 64, 2, true>(a, s);
    }
  }
  switch (c.fmt) {
    case kQ4_0: e = launch_up_npl<kQ4_0>(a, n_items_max, s); break;
    case kQ8_0: e = launch_up_npl<kQ8_0>(a, n_items_max, s); break;
    case kIQ4_NL: e = launch_up_npl<kIQ4_NL>(a, n_items_max, s); break;
    case kQ4_K: e = launch_up_npl<kQ4_K>(a, n_items_max, s); break;
    case kQ6_K: e = launch_up_npl<kQ6_K>(a, n_items_max, s); break;
    case kQ5_K: e = launch_up_npl<kQ5_K>(a, n_items_max, s); break;
    case kIQ4_XS: e = launch_up_npl<kIQ4_XS>(a, n_items_max, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // The down launch picks its rows per item and the tile size for them.
  const MoeFusedArgs& d = a;
  switch (c.fmt) {
#define QG_DN(F)                                                           \
  case F:                                                                  \
    switch (U) {                                                           \
      case 16: return launch_dn_t<F, 16, 1>(d, s);                         \
      case 32: return launch_dn_t<F, 32, 1>(d, s);                         \
      case 64: return launch_dn_t<F, 64, 1>(d, s);                         \
      default: return launch_dn_t<F, 64, 2>(d, s);                         \
    }
    QG_DN(kQ4_0)
    QG_DN(kQ8_0)
    QG_DN(kIQ4_NL)
    QG_DN(kQ4_K)
    QG_DN(kQ6_K)
    QG_DN(kQ5_K)
    QG_DN(kIQ4_XS)
#undef QG_DN
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
