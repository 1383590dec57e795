// Row GEMV over packed block-quantized weights, m <= 16 tokens (gfx950).
//
// The weights are read once, in their packed block form, with no fp16 or
// int8 expansion of the matrix; each block is decoded in registers and
// multiplied with int8 activation blocks by 4-way int8 dot products, then
// scaled. K-quant super-blocks apply their scale and min correction terms and
// the non-linear 4-bit format looks its codes up in a 16-entry codebook held
// in registers ("Why expert caching can't save dense models", xhh.club, Q&A
// on computing GGUF blocks without FP16 expansion). The memory-access
// granularity is what decides speed for this bandwidth-bound kernel ("01 ·
// Phase overview: from 2B to 8B to MoE", icman.com.cn, ledger item ㉑).
//
// Kernel structure (one design for all five formats):
//  * A workgroup is 4 waves. At start it stages the quantized activations
//    of all its tokens in LDS, in a layout that makes each lane's 32-element
//    unit a conflict-free 16-byte read: per token, the first 16 codes of
//    every unit, then the last 16 codes of every unit, then (dx, packed
//    16-element sums) per unit.
//  * Each wave then walks "steps": a step is G whole rows (short rows) or one
//    K-segment of one row (long rows) -- a contiguous byte range of the
//    matrix. The wave loads the range with fully coalesced 128-bit loads
//    (lane l takes 16-byte chunks l, l+64, ...) into registers one step
//    ahead, writes it to a wave-private LDS buffer, and decodes from there:
//    blocks of 18, 34 and 210 bytes are not 16-byte aligned, so the LDS hop
//    turns the coalesced byte stream into per-lane block views.
//  * Lane l owns 32-element units l % LPR + LPR * j of row l / LPR within a
//    pass (LPR = lanes per row, 64 when K >= 2048). Each lane keeps fp32
//    partial sums per row; the LPR lanes of a row are summed by a butterfly
//    and one lane stores y. No atomics: results are bitwise reproducible.
#include "common.cuh"
#include "formats.cuh"
#include "internal.h"

namespace qg {

#ifndef QG_TILE_CAP
#define QG_TILE_CAP 0     // > 0: one step-size cap for every format (tuning)
#endif
#ifndef QG_WGS_PER_CU
#define QG_WGS_PER_CU 5   // cap on resident workgroups per CU for one matrix (measured on Q8_0)
#endif

#ifndef QG_BALANCE
#define QG_BALANCE 0      // 1: size the grid so every wave gets the same step count
#endif
#ifndef QG_WLOAD_AUX
#define QG_WLOAD_AUX 2    // cache-policy bits of the weight loads (2: non-temporal, read once)
#endif
#ifndef QG_Q4K_DIRECT
#define QG_Q4K_DIRECT 1   // single-token Q4_K, Q5_K and IQ4_XS GEMVs use the register-direct kernel
#endif
#ifndef QG_PREFETCH
#define QG_PREFETCH 1     // weight steps in flight per wave (1 or 2)
#endif
#ifndef QG_WAVES_PER_WG
#define QG_WAVES_PER_WG 4
#endif
#ifndef QG_FUSED_WAVES
#define QG_FUSED_WAVES 16   // waves per workgroup when the kernel quantizes x itself
#endif
#ifndef QG_FUSED_WGS_PER_CU
#define QG_FUSED_WGS_PER_CU 1
#endif

constexpr int kWavesPerWG = QG_WAVES_PER_WG;
// With the quantizer in the prologue every workgroup quantizes all of x, so
// fewer, larger workgroups quantize it fewer times (measured on MI355X at
// K = 4096: 16 waves, one workgroup per CU).
template <bool FUSEQ> constexpr int waves_per_wg() { return FUSEQ ? QG_FUSED_WAVES : kWavesPerWG; }
// Packed bytes per step (max), per format. Measured on MI355X: smaller steps
// give each wave more steps (a shorter pipeline tail after its last load)
// and leave LDS for more resident waves; below ~2.5 KB the per-step overhead
// wins. Q8_0 rows (4352 B at K=4096) are then split into K-segments. IQ4_NL
// is bound by its codebook arithmetic, not by the loads: four 2304-byte rows
// per step spread the per-step row sums over more blocks (lm_head 4096 ->
// 248320: 119.0 -> 116.9 us sustained).
constexpr int tile_cap(int fmt) {
  return QG_TILE_CAP > 0 ? QG_TILE_CAP
         : fmt == kQ8_0 ? 2560 : fmt == kQ4_K ? 5120 : fmt == kQ5_K ? 5632
         : fmt == kIQ4_NL ? 9216 : fmt == kIQ4_XS ? 4608 : 3584;
}
// 16-byte chunks a step can span (alignment adds up to two), per lane.
template <int FMT> constexpr int loads_per_lane() { return (tile_cap(FMT) + 32 + 1023) / 1024; }
constexpr int kLdsLimit = kLdsBytes;
// Word 3 of a raw (unswizzled, unformatted) buffer resource on gfx9-family
// GPUs, gfx950 included.
constexpr int kBufferDword3 = 0x00020000;

// ------------------------------------------------------------ the kernel --

struct GemvGeom {
  int U;          // 32-element units per row
  int LPR, RPP;   // lanes per row, rows per pass
  int lpr_log;    // log2(LPR)
  int SU;         // units per step segment (== U when rows are whole)
  int nseg;       // segments per row
  int64_t rb;     // row bytes
  int64_t nrowtiles;
  int act_bytes;  // LDS bytes of staged activations
  int tile_buf;   // LDS bytes of one wave's step buffer
};

struct GemvArgs {
  GemvProblem p;
  GemvGeom g;
};

template <typename F>
QG_DEV int64_t seg_bytes(int units) { return (int64_t)(units / F::kUPB) * F::kBB; }

// Stage the quantized activations of tokens t < mcnt in LDS. From int8 codes
// (xq/dx) or, with FUSEQ, by quantizing fp32 x here: eight lanes per 32-element
// unit, the same arithmetic as the standalone quantizer. Token slots past
// mcnt are never read, so they are not staged.
// The first batch of token 0's staging input, loaded before the first
// weight step is requested: vector loads return in issue order, so inputs
// requested after the weights could only be used once the weights arrived.
struct StagePre {
  float4 v[4];   // FUSEQ: fp32 x, tasks threadIdx.x + r * blockDim.x
  int4 lo, hi;   // otherwise: codes of unit threadIdx.x
  float d;
};

template <bool DOTS, bool FUSEQ>
QG_DEV void stage_prefetch(StagePre& pre, const GemvProblem& p, int U, int64_t ar) {
  if constexpr (FUSEQ) {
    const float4* xr = reinterpret_cast<const float4*>(p.xf + ar * p.xs);
    const int ntask = U * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = threadIdx.x + r * blockDim.x;
      pre.v[r] = i < ntask ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
    const int u = threadIdx.x;
    if (u < U) {
      const int4* src = reinterpret_cast<const int4*>(p.xq + ar * p.xs);
      pre.lo = src[2 * u];
      pre.hi = src[2 * u + 1];
      pre.d = DOTS ? 0.0f : p.dx[ar * (p.xs / 32) + u];
    }
  }
}

template <int MT, bool DOTS, bool FUSEQ, typename RowFn>
QG_DEV void stage_activations(uint8_t* smem, const GemvProblem& p, int U, int mcnt, RowFn out_row,
                              bool write_back, const StagePre& pre) {
  const int tokb = act_token_bytes(U);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t >= mcnt) break;
    const int64_t ar = out_row(t) / p.act_div;  // 32-bit operands: slot rows are small
    uint8_t* tok = smem + t * tokb;
    if constexpr (FUSEQ) {
      // Batches of 4 tasks per thread: all loads of a batch are issued
      // before any is used, so the batch costs one memory round trip.
      const float4* xr = reinterpret_cast<const float4*>(p.xf + ar * p.xs);
      const int ntask = U * 8;
      for (int base = threadIdx.x; base < ntask; base += 4 * blockDim.x) {
        float4 vb[4];
        if (t == 0 && base == (int)threadIdx.x) {
#pragma unroll
          for (int r = 0; r < 4; ++r) vb[r] = pre.v[r];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = base + r * blockDim.x;
            vb[r] = i < ntask ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = base + r * blockDim.x;
          if (i < ntask) {  // whole 8-lane groups are in or out together
            const float4 v = vb[r];
            const int u = i >> 3, part = i & 7;
            const float a = max8(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            const float d = (a > 0.0f) ? a / 127.0f : 0.0f;
            int s;
            const uint32_t packed = q8_pack4(v, d, s);
            s = sum4(s);                          // lanes 0-3: sum of codes 0..15; 4-7: 16..31
            const int other = other_quad(s);
            if (part < 4) *reinterpret_cast<uint32_t*>(tok + 16 * u + 4 * part) = packed;
            else *reinterpret_cast<uint32_t*>(tok + 16 * U + 16 * u + 4 * (part - 4)) = packed;
            if (part == 0)
              *reinterpret_cast<int2*>(tok + 32 * U + 8 * u) =
                  make_int2(__float_as_int(d), (s & 0xffff) | (other << 16));
            if (write_back) {
              reinterpret_cast<uint32_t*>(p.xq_out + ar * p.xs)[i] = packed;
              if (part == 0) {
                p.dx_out[ar * (p.xs / 32) + u] = d;
                if (p.sx_out) p.sx_out[ar * (p.xs / 32) + u] = s + other;
              }
            }
          }
        }
      }
    } else {
      const int4* src = reinterpret_cast<const int4*>(p.xq + ar * p.xs);
      const float* dxr = DOTS ? nullptr : p.dx + ar * (p.xs / 32);
      for (int u = threadIdx.x; u < U; u += blockDim.x) {
        int4 lo, hi;
        float d = 0.0f;
        if (t == 0 && u == (int)threadIdx.x) {
          lo = pre.lo;
          hi = pre.hi;
          d = pre.d;
        } else {
          lo = src[2 * u];
          hi = src[2 * u + 1];
          if constexpr (!DOTS) d = dxr[u];
        }
        const int ones = 0x01010101;
        const int sa = dot4(lo.x, ones, dot4(lo.y, ones, dot4(lo.z, ones, dot4(lo.w, ones, 0))));
        const int sb = dot4(hi.x, ones, dot4(hi.y, ones, dot4(hi.z, ones, dot4(hi.w, ones, 0))));
        *reinterpret_cast<int4*>(tok + 16 * u) = lo;
        *reinterpret_cast<int4*>(tok + 16 * U + 16 * u) = hi;
        *reinterpret_cast<int2*>(tok + 32 * U + 8 * u) = make_int2(__float_as_int(d), (sa & 0xffff) | (sb << 16));
      }
    }
  }
}

// FMT: block format; MT: token slots (activations staged per workgroup);
// P: row passes per step (compile time, so every pass's LDS reads are issued
// before any pass's arithmetic); DOTS: integer-store checking epilogue;
// FUSEQ: quantize fp32 activations in the prologue.
template <int FMT, int MT, int P, bool DOTS, bool FUSEQ>
__global__ __launch_bounds__(waves_per_wg<FUSEQ>() * 64) void gemv_kernel(const GemvArgs args) {
  constexpr int kWPG = waves_per_wg<FUSEQ>();
  using F = typename FmtOf<FMT>::T;
  extern __shared__ __align__(16) uint8_t smem[];
  const GemvProblem& p = args.p;
  const GemvGeom& g = args.g;
  const int prob = blockIdx.y;

  // Resolve this problem's matrix, token count and row mapping.
  const uint8_t* W = p.w;
  int mcnt = p.m;
  const int32_t* rows = nullptr;  // grouped mode: output (slot) row of each token
  bool shared = false;
  if (p.tbl) {
    if (prob >= p.tbl[0]) return;  // whole workgroup leaves before any barrier
    const int32_t* e = p.tbl + 1 + (int64_t)prob * p.tbl_stride;
    shared = e[0] < 0;
    W = shared ? p.w_shared : p.w + (int64_t)e[0] * p.w_stride;
    mcnt = e[1];
    rows = e + 2;
  }
  auto out_row = [&](int t) __attribute__((always_inline)) -> int { return p.tbl ? rows[t] : t; };

  const int U = g.U;
  const int tokb = act_token_bytes(U);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  uint8_t* tile = smem + g.act_bytes + wid * g.tile_buf;
  const int64_t nwaves = (int64_t)gridDim.x * kWPG;
  const int LPR = g.LPR, RPP = g.RPP;  // powers of two: use shifts, not divisions
  const int lpr_log = g.lpr_log, rpp_log = 6 - g.lpr_log;
  const int lam = lane & (LPR - 1);
  const int rho = lane >> lpr_log;
  const int G = P * RPP;

  // Byte range of step (rt, seg), relative to W.
  auto step_range = [&](int64_t rt, int seg, int64_t& b0, int64_t& b1) __attribute__((always_inline)) {
    const int64_t r0 = rt * G;
    const int64_t nrows = (p.n - r0) < G ? (p.n - r0) : G;
    if (g.nseg == 1) {
      b0 = r0 * g.rb;
      b1 = (r0 + nrows) * g.rb;
    } else {
      const int u0 = seg * g.SU;
      const int su = (U - u0) < g.SU ? (U - u0) : g.SU;
      b0 = r0 * g.rb + seg_bytes<F>(u0);
      b1 = b0 + seg_bytes<F>(su);
    }
  };

  // This wave's steps: row tiles rt_first + i * nwaves, each in nseg
  // K-segments. One register buffer holds the next step while the current
  // one is decoded from LDS.
  const int64_t rt_first = (int64_t)blockIdx.x * kWPG + wid;
  constexpr int kLPL = loads_per_lane<FMT>();
  // Loads go through a buffer resource that spans exactly the step's 16-byte
  // chunks: lanes past the end (and a whole wave past the last step) read
  // zeros with no memory access. Every load is issued unconditionally, so the
  // compiler can wait for earlier loads without draining these.
  auto issue = [&](u32x4(&buf)[kLPL], int64_t rt, int seg) __attribute__((always_inline)) {
    const bool ok = rt < g.nrowtiles;
    int64_t b0 = 0, b1 = 0;
    if (ok) step_range(rt, seg, b0, b1);
    const int64_t a0 = b0 & ~(int64_t)15;
    const int nch = ok ? (int)((((b1 + 15) & ~(int64_t)15) - a0) >> 4) : 0;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W + a0), 0, nch * 16, kBufferDword3);
#pragma unroll
    for (int i = 0; i < kLPL; ++i)
      buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + kWave * i) * 16, 0, QG_WLOAD_AUX);
  };
  // Staging input first, then the first weight step: both round trips
  // overlap, and the staging arithmetic runs while the weights are in flight.
  StagePre pre;
  if (mcnt > 0) stage_prefetch<DOTS, FUSEQ>(pre, p, U, out_row(0) / p.act_div);
  // The step after (rt, seg) in this wave's sequence.
  auto next_step = [&](int64_t rt, int seg, int64_t& rt2, int& seg2) __attribute__((always_inline)) {
    rt2 = rt;
    seg2 = seg + 1;
    if (seg2 == g.nseg) { seg2 = 0; rt2 = rt + nwaves; }
  };
  u32x4 bufA[kLPL];
  issue(bufA, rt_first, 0);
#if QG_PREFETCH > 1
  // A second step in flight while the first is decoded.
  u32x4 bufB[kLPL];
  int64_t rtn;
  int segn;
  next_step(rt_first, 0, rtn, segn);
  issue(bufB, rtn, segn);
#endif

  // With fused quantization, workgroup 0 of the plain problem (or of each
  // shared-expert entry, which together cover every token once) stores the
  // activation codes in the workspace.
  stage_activations<MT, DOTS, FUSEQ>(smem, p, U, mcnt, out_row,
                                     FUSEQ && p.xq_out && blockIdx.x == 0 && (!p.tbl || shared), pre);
  __syncthreads();

  // Codebook pool words, pinned in registers (opaque values): the byte
  // permutes then take them as register operands without re-copying them
  // from scalar registers.
  uint32_t cbr[4] = {p.cb[0], p.cb[1], p.cb[2], p.cb[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(cbr[i]));

  float acc[P][MT];
#pragma unroll
  for (int a = 0; a < P; ++a)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[a][t] = 0.0f;

  // One step: move its bytes from registers to the wave's LDS buffer, reuse
  // the registers for step (rtq, segq), then decode and accumulate.
  auto process = [&](u32x4(&buf)[kLPL], int64_t rt, int seg, int64_t rtq, int segq) __attribute__((always_inline)) {
    int64_t b0, b1;
    step_range(rt, seg, b0, b1);
    const int64_t a0 = b0 & ~(int64_t)15;
    {
      const int nch = (int)((((b1 + 15) & ~(int64_t)15) - a0) >> 4);
#pragma unroll
      for (int i = 0; i < kLPL; ++i) {
        const int c = lane + kWave * i;
        if (c < nch) *reinterpret_cast<u32x4*>(tile + 16 * c) = buf[i];
      }
    }
    issue(buf, rtq, segq);

    // ---- decode this step from LDS and accumulate
    const int64_t r0 = rt * G;
    const int nrows = (int)((p.n - r0) < G ? (p.n - r0) : G);
    const int u0 = seg * g.SU;
    const int su = (U - u0) < g.SU ? (U - u0) : g.SU;
    const uint32_t base = (uint32_t)(b0 - a0);  // LDS offset of the step's first byte
    const int jmax = (su + LPR - 1) >> lpr_log;
    for (int j = 0; j < jmax; ++j) {
      const int ul = lam + LPR * j;
      if (ul < su) {
        const int ug = u0 + ul;
        const uint32_t uoff = (uint32_t)((ul / F::kUPB) * F::kBB);
        const int sub = ul % F::kUPB;
        // All passes' weight units first (independent LDS reads in flight
        // together); rows past the end re-read the last valid row and are
        // never stored.
        typename F::W wv[P];
#pragma unroll
        for (int pp = 0; pp < P; ++pp) {
          int rl = pp * RPP + rho;
          rl = rl < nrows ? rl : nrows - 1;
          wv[pp] = F::load(tile, base + (uint32_t)(rl * g.rb) + uoff, sub, cbr);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < mcnt) {  // wave-uniform: skips padded tokens
            const Act a = load_act(smem + t * tokb, U, ug);
#pragma unroll
            for (int pp = 0; pp < P; ++pp) {
              if constexpr (DOTS) {
                const int rl = pp * RPP + rho;
                if (rl < nrows) {
                  int32_t* o = p.dots + ((int64_t)out_row(t) * p.n + r0 + rl) * ((int64_t)U * F::kDotsPerUnit) +
                               (int64_t)ug * F::kDotsPerUnit;
                  F::dots(wv[pp], a, o);
                }
              } else {
                acc[pp][t] = F::fma(wv[pp], a, acc[pp][t]);
              }
            }
          }
        }
      }
    }

    if (!DOTS && seg == g.nseg - 1) {
      // Row sums: lanes of a group add up; lane pp*RPP + rho then holds row
      // r0 + pp*RPP + rho, so each token's rows go out in one store.
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t < mcnt) {
          float outv = 0.0f;
          auto per_row = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int pp = 0; pp < P; ++pp) {
              const float sum = group_sum(acc[pp][t], LPR);
              float v;
              if (RPP == 1) v = sum;
              else v = __shfl(sum, (lane & (RPP - 1)) << lpr_log, kWave);
              if ((lane >> rpp_log) == pp) outv = v;
            }
          };
          if constexpr (P == 4) {
            // A whole wave per row: the four rows are reduced together.
            if (LPR == kWave) outv = rows4_wave_sum(acc[0][t], acc[1][t], acc[2][t], acc[3][t], lane);
            else per_row();
          } else {
            per_row();
          }
#pragma unroll
          for (int pp = 0; pp < P; ++pp) acc[pp][t] = 0.0f;
          if (lane < nrows) p.y[(int64_t)out_row(t) * p.ldy + r0 + lane] = outv;
        }
      }
    }
  };

  int64_t rt = rt_first;
  int seg = 0;
#if QG_PREFETCH > 1
  // bufA holds (rt, seg), bufB the step after it; each buffer is refilled
  // with the step two ahead as soon as it has been copied to LDS.
  while (rt < g.nrowtiles) {
    int64_t rt3;
    int seg3;
    next_step(rtn, segn, rt3, seg3);
    process(bufA, rt, seg, rt3, seg3);
    rt = rtn; seg = segn; rtn = rt3; segn = seg3;
    if (rt >= g.nrowtiles) break;
    next_step(rtn, segn, rt3, seg3);
    process(bufB, rt, seg, rt3, seg3);
    rt = rtn; seg = segn; rtn = rt3; segn = seg3;
  }
#else
  while (rt < g.nrowtiles) {
    int64_t rt2;
    int seg2;
    next_step(rt, seg, rt2, seg2);
    process(bufA, rt, seg, rt2, seg2);
    rt = rt2;
    seg = seg2;
  }
#endif
}

// ------------------------------------------------------------- launchers --

int fmt_block_elems(int fmt) {
  switch (fmt) {
    case kQ4_0: case kQ8_0: case kIQ4_NL: return 32;
    case kQ4_K: case kQ6_K: case kQ5_K: case kIQ4_XS: return 256;
    case kF32: return 1;
    default: return 0;
  }
}

int fmt_block_bytes(int fmt) {
  switch (fmt) {
    case kQ4_0: case kIQ4_NL: return 18;
    case kQ8_0: return 34;
    case kQ4_K: return 144;
    case kQ6_K: return 210;
    case kQ5_K: return 176;
    case kIQ4_XS: return 136;
    case kF32: return 4;
    default: return 0;
  }
}

int64_t fmt_row_bytes(int fmt, int64_t k) {
  const int be = fmt_block_elems(fmt);
  if (be <= 0 || k <= 0 || k % be) return -1;
  return k / be * fmt_block_bytes(fmt);
}

static int floor_pow2(int v) {
  int r = 1;
  while (r * 2 <= v) r *= 2;
  return r;
}

// Largest passes-per-step the kernels are instantiated for, per token tile.
static int max_passes(int mt) { return mt <= 2 ? 8 : mt == 4 ? 4 : mt == 8 ? 2 : 1; }

// Choose the step geometry for a format, shape and token tile; returns P.
// nprob: problems sharing the launch (grouped mode), which together spread
// over the chip.
static int plan_geom(int fmt, int64_t n, int64_t k, int MT, bool dots, bool fused, int nprob, GemvGeom& g) {
  g = GemvGeom{};
  const int upb = fmt_block_elems(fmt) / 32;
  const int bb = fmt_block_bytes(fmt);
  g.U = (int)(k / 32);
  g.rb = fmt_row_bytes(fmt, k);
  g.LPR = g.U >= kWave ? kWave : floor_pow2(g.U);
  g.RPP = kWave / g.LPR;
  g.lpr_log = 0;
  while ((1 << g.lpr_log) < g.LPR) ++g.lpr_log;
  int P = 1;
  const int cap = tile_cap(fmt);
  if (g.rb * g.RPP <= cap) {
    g.nseg = 1;
    g.SU = g.U;
    // Fused-quantizer instances run 16 waves per workgroup (128 registers
    // per lane): at most 4 passes, more would spill.
    const int pm = dots ? 1 : (fused && max_passes(MT) > 4 ? 4 : max_passes(MT));
    while (P * 2 <= pm && g.rb * g.RPP * P * 2 <= cap) P *= 2;
    // Keep enough steps to spread the matrix over the whole chip.
    const int64_t want_waves = (int64_t)device_cus() * 8;
    while (P > 1 && nprob * ((n + (int64_t)P * g.RPP - 1) / ((int64_t)P * g.RPP)) < want_waves) P >>= 1;
  } else {
    // Long rows: one row per step, split into K-segments of whole
    // super-blocks that are a multiple of 64 units.
    const int64_t unit_bytes_x64 = (int64_t)64 * bb / upb;  // bytes of 64 units
    int su = (int)(cap / unit_bytes_x64) * 64;
    if (su < 64) su = 64;
    g.SU = su;
    g.nseg = (g.U + su - 1) / su;
  }
  const int64_t G = (int64_t)P * g.RPP;
  g.nrowtiles = (n + G - 1) / G;
  g.act_bytes = MT * act_token_bytes(g.U);
  const int64_t step_max = g.nseg == 1 ? G * g.rb : (int64_t)(g.SU / upb) * bb;
  g.tile_buf = (int)((step_max + 32 + 15) / 16 * 16 + 16);  // + alignment chunks + over-read
  // A step's 16-byte chunks (two more for alignment) must fit the per-lane
  // register buffer the kernel is compiled with.
  if ((step_max + 15) / 16 + 2 > (int64_t)kWave * ((cap + 32 + 1023) / 1024)) return 0;
  return P;
}

template <int FMT, int MT, int P, bool DOTS, bool FUSEQ>
static hipError_t launch_t(const GemvArgs& a, hipStream_t s) {
  auto kern = gemv_kernel<FMT, MT, P, DOTS, FUSEQ>;
  constexpr int kWPG = waves_per_wg<FUSEQ>();
  const size_t lds = (size_t)a.g.act_bytes + (size_t)kWPG * a.g.tile_buf;
  // Persistent grid: no more workgroups than can be resident at once, so
  // every wave walks its share of the steps without a second launch round.
  // Resident workgroups per CU depend on the LDS size (activations vary with
  // K); the answer is cached per kernel, LDS size and device.
  int per_cu = 0, cus = 0;
  hipError_t qe = kernel_residency(reinterpret_cast<const void*>(kern), kWPG * 64, lds, true, &per_cu, &cus);
  if (qe != hipSuccess) return qe;
  // A single matrix streams best with fewer resident workgroups than fit;
  // grouped launches (many small problems) use all of them.
  const int cap = FUSEQ ? QG_FUSED_WGS_PER_CU : QG_WGS_PER_CU;
  if (a.p.nprob == 1 && cap > 0 && cap < per_cu) per_cu = cap;
  // Waves available to each problem, then the fewest waves that still give
  // every wave the same number of row tiles (ceil), so no wave runs a
  // lone extra step at the end.
  // Grouped launches split the resident waves among their problems.
  const int64_t cap_waves = (int64_t)cus * per_cu * kWPG;
  int64_t wmax = cap_waves / a.p.nprob;
  if (wmax < kWPG) wmax = kWPG;
#if QG_BALANCE
  const int64_t per_wave = (a.g.nrowtiles + wmax - 1) / wmax;
  const int64_t waves = (a.g.nrowtiles + per_wave - 1) / per_wave;
#else
  const int64_t waves = a.g.nrowtiles < wmax ? a.g.nrowtiles : wmax;
#endif
  int64_t wgs = (waves + kWPG - 1) / kWPG;
  // Grouped launches: never more workgroups than fit at once in all, so no
  // problem waits for a second round.
  if (a.p.nprob > 1) {
    int64_t fit = cap_waves / kWPG / a.p.nprob;
    if (fit < 1) fit = 1;
    if (wgs > fit) wgs = fit;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs, (unsigned)a.p.nprob), dim3(kWPG * 64), lds, s, a);
  return hipGetLastError();
}

template <int FMT, int MT, bool DOTS, bool FUSEQ>
static hipError_t launch_p(const GemvArgs& a, int P, hipStream_t s) {
  if constexpr (DOTS) {
    return launch_t<FMT, MT, 1, true, false>(a, s);
  } else {
    switch (P) {
      case 8: if constexpr (MT <= 2 && !FUSEQ) return launch_t<FMT, MT, 8, false, FUSEQ>(a, s); break;
      case 4: if constexpr (MT <= 4) return launch_t<FMT, MT, 4, false, FUSEQ>(a, s); break;
      case 2: if constexpr (MT <= 8) return launch_t<FMT, MT, 2, false, FUSEQ>(a, s); break;
      default: break;
    }
    return launch_t<FMT, MT, 1, false, FUSEQ>(a, s);
  }
}

template <int FMT, bool DOTS, bool FUSEQ>
static hipError_t launch_mt(const GemvArgs& a, int mt, int P, hipStream_t s) {
  switch (mt) {
    case 1: return launch_p<FMT, 1, DOTS, FUSEQ>(a, P, s);
    case 2: return launch_p<FMT, 2, DOTS, FUSEQ>(a, P, s);
    case 4: return launch_p<FMT, 4, DOTS, FUSEQ>(a, P, s);
    case 8: return launch_p<FMT, 8, DOTS, FUSEQ>(a, P, s);
    default: return launch_p<FMT, 16, DOTS, FUSEQ>(a, P, s);
  }
}

template <bool DOTS, bool FUSEQ>
static hipError_t launch_fmt(int fmt, const GemvArgs& a, int mt, int P, hipStream_t s) {
  switch (fmt) {
    case kQ4_0: return launch_mt<kQ4_0, DOTS, FUSEQ>(a, mt, P, s);
    case kQ8_0: return launch_mt<kQ8_0, DOTS, FUSEQ>(a, mt, P, s);
    case kQ4_K: return launch_mt<kQ4_K, DOTS, FUSEQ>(a, mt, P, s);
    case kQ6_K: return launch_mt<kQ6_K, DOTS, FUSEQ>(a, mt, P, s);
    case kIQ4_NL: return launch_mt<kIQ4_NL, DOTS, FUSEQ>(a, mt, P, s);
    case kQ5_K: return launch_mt<kQ5_K, DOTS, FUSEQ>(a, mt, P, s);
    case kIQ4_XS: return launch_mt<kIQ4_XS, DOTS, FUSEQ>(a, mt, P, s);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_any(int fmt, const GemvArgs& a, int mt, int P, bool dots, hipStream_t s) {
  if (dots) return launch_fmt<true, false>(fmt, a, mt, P, s);
  if (a.p.xf) return launch_fmt<false, true>(fmt, a, mt, P, s);
  return launch_fmt<false, false>(fmt, a, mt, P, s);
}

static int token_tile(int m) {
  if (m <= 1) return 1;
  if (m <= 2) return 2;
  if (m <= 4) return 4;
  if (m <= 8) return 8;
  return 16;
}

hipError_t launch_gemv(int fmt, const GemvProblem& p, bool dots_epilogue, hipStream_t s) {
  if (p.m < 1 || p.m > kGemvMaxTokens || p.n < 1) return hipErrorInvalidValue;
  if (p.xf && dots_epilogue) return hipErrorInvalidValue;
#if QG_Q4K_DIRECT
  if (kdirect_ok(fmt, p, dots_epilogue)) return launch_kdirect(fmt, p, dots_epilogue, s);
#endif
  int mt = token_tile(p.tbl ? kGroupTokens : p.m);
  GemvArgs a;
  a.p = p;
  int P = plan_geom(fmt, p.n, p.k, mt, dots_epilogue, p.xf != nullptr, p.tbl ? p.nprob : 1, a.g);
  const size_t wpg = p.xf ? (size_t)waves_per_wg<true>() : (size_t)waves_per_wg<false>();
  // Keep the staged activations within LDS; fall back to smaller token tiles.
  while ((size_t)a.g.act_bytes + wpg * a.g.tile_buf > (size_t)kLdsLimit && mt > 1) {
    mt >>= 1;
    P = plan_geom(fmt, p.n, p.k, mt, dots_epilogue, p.xf != nullptr, p.tbl ? p.nprob : 1, a.g);
  }
  if (P == 0 || (size_t)a.g.act_bytes + wpg * a.g.tile_buf > (size_t)kLdsLimit)
    return hipErrorInvalidValue;
  if (p.tbl && mt < kGroupTokens) return hipErrorInvalidValue;  // entries cannot be split
  if (mt >= p.m || p.tbl) return launch_any(fmt, a, mt, P, dots_epilogue, s);
  // Token chunks of mt.
  for (int t0 = 0; t0 < p.m; t0 += mt) {
    GemvArgs c = a;
    c.p.m = (p.m - t0) < mt ? (p.m - t0) : mt;
    if (p.xf) c.p.xf = p.xf + (int64_t)t0 * p.xs;
    if (p.xq) c.p.xq = p.xq + (int64_t)t0 * p.xs;
    if (p.dx) c.p.dx = p.dx + (int64_t)t0 * (p.xs / 32);
    if (p.xq_out) c.p.xq_out = p.xq_out + (int64_t)t0 * p.xs;
    if (p.dx_out) c.p.dx_out = p.dx_out + (int64_t)t0 * (p.xs / 32);
    if (p.sx_out) c.p.sx_out = p.sx_out + (int64_t)t0 * (p.xs / 32);
    if (p.y) c.p.y = p.y + (int64_t)t0 * p.ldy;
    if (p.dots) c.p.dots = p.dots + (int64_t)t0 * p.n * (p.k / (fmt == kQ6_K ? 16 : 32));
    hipError_t e = launch_any(fmt, c, mt, P, dots_epilogue, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qg
