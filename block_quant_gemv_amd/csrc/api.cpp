// C-ABI layer: plan validation, workspace layout and kernel launches.
//
// Every entry point validates its arguments on the host before it enqueues
// anything, returns a status code and never aborts, throws or prints -- the
// convention of the pure-C device module in "01 · Phase overview: from 2B to
// 8B to MoE" (icman.com.cn, section 一 and ledger item ①), without its CPU
// fallback: an error is reported, never silently degraded (the same page's
// ledger item ⑤ on explicit warnings instead of silent slowdowns).
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "../../include/qattn.h"
#include "../../include/qgemv.h"
#include "internal.h"
#include "attn.h"
#include "moe.h"
#include "s16.h"
#include "fact.h"
#include "mfma.h"
#include "swiglu.h"

using namespace qg;

struct qgemv_plan {
  qgemv_desc d;
  int8_t cb[16];
  uint32_t cbw[4];  // cb as the device's two byte-permute pools (codebook_pools)
};

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool is_block_fmt(int f) { return f >= QFMT_Q4_0 && f <= QFMT_IQ4_XS; }

bool has_codebook(int f) { return f == QFMT_IQ4_NL || f == QFMT_IQ4_XS; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Byte-permute pools of a 16-entry int8 codebook T for the device lookup:
// pool L (words 0, 1) answers codes 0..7 at selector n, pool H (words 2, 3)
// codes 8..15 at selector n ^ 8, and the device takes the xor of the two
// permutes. A selector in 8..15 makes the permute yield a fill byte: the
// sign of pool byte 1, 3, 5 or 7 spread over the byte for 8..11, 0x00 for
// 12, 0xFF for 13..15. Each pool byte is stored xor-ed with the fill that
// its code meets in the other pool. The fills of 8..11 depend on pool bytes
// computed here; those chains end at bytes 4..7 (constant fills) within
// three links, so four sweeps settle every byte. The final loop decodes all
// 16 codes the way the device does and checks them against T.
bool codebook_pools(const int8_t* T, uint32_t* w) {
  uint8_t L[8] = {0}, H[8] = {0};
  auto fill = [](const uint8_t* pool, int sel) -> uint8_t {  // sel in 8..15
    if (sel >= 13) return 0xFF;
    if (sel == 12) return 0x00;
    return (pool[2 * (sel - 8) + 1] & 0x80u) ? 0xFF : 0x00;
  };
  for (int sweep = 0; sweep < 4; ++sweep)
    for (int n = 0; n < 8; ++n) {
      L[n] = (uint8_t)((uint8_t)T[n] ^ fill(H, n + 8));      // code n: H's selector is n + 8
      H[n] = (uint8_t)((uint8_t)T[n + 8] ^ fill(L, n + 8));  // code n + 8: L's selector is n + 8
    }
  for (int c = 0; c < 16; ++c) {
    const int hs = c ^ 8;
    const uint8_t lo = c < 8 ? L[c] : fill(L, c);
    const uint8_t hi = hs < 8 ? H[hs] : fill(H, hs);
    if ((int8_t)(lo ^ hi) != T[c]) return false;
  }
  memcpy(w, L, 8);
  memcpy(w + 2, H, 8);
  return true;
}

// Named regions of a workspace, in order, each 256-byte aligned.
struct Region { const char* name; size_t bytes; };

struct Layout {
  Region r[24];
  int n = 0;
  void add(const char* name, size_t bytes) { r[n++] = Region{name, bytes}; }
  size_t offset(const char* name, bool* found) const {
    size_t off = 0;
    for (int i = 0; i < n; ++i) {
      if (strcmp(r[i].name, name) == 0) { *found = true; return off; }
      off += round_up(r[i].bytes, 256);
    }
    *found = false;
    return 0;
  }
  size_t total() const {
    size_t off = 0;
    for (int i = 0; i < n; ++i) off += round_up(r[i].bytes, 256);
    return off;
  }
};

Layout layout_of(const qgemv_plan* h, int m) {
  Layout L;
  const qgemv_desc& d = h->d;
  if (d.kind == QKIND_GEMV) {
    L.add("xq", (size_t)m * d.k);
    L.add("dx", (size_t)m * (d.k / 32) * 4);
    L.add("sx", (size_t)m * (d.k / 32) * 4);
    if (m >= kMfmaMinTokens) {
      // token-tiled codes for the batched matrix-core path, written by the
      // quantizer for every plan so that plans with the same k share a
      // quantized workspace
      L.add("xqt", gemm32_tiled_act_bytes(d.k));
      L.add("dxt", (size_t)(d.k / 32) * 32 * 4);
      L.add("cxt", (size_t)(d.k / 32) * 32 * 4);
    }
  } else if (d.kind == QKIND_FFN) {
    L.add("xq", (size_t)m * d.hidden);
    L.add("dx", (size_t)m * (d.hidden / 32) * 4);
    L.add("sx", (size_t)m * (d.hidden / 32) * 4);
    L.add("gu", (size_t)m * 2 * d.inter * 4);
    L.add("h", (size_t)m * d.inter * 4);
    L.add("hq", (size_t)m * d.inter);
    L.add("hd", (size_t)m * (d.inter / 32) * 4);
    L.add("hs", (size_t)m * (d.inter / 32) * 4);
  } else {
    const size_t slots = (size_t)m * (d.top_k + 1);
    L.add("logits", (size_t)m * d.n_experts * 4);
    L.add("ids", (size_t)m * d.top_k * 4);
    L.add("wts", (size_t)m * d.top_k * 4);
    L.add("xq", (size_t)m * d.hidden);
    L.add("dx", (size_t)m * (d.hidden / 32) * 4);
    L.add("sx", (size_t)m * (d.hidden / 32) * 4);
    L.add("gu", slots * 2 * d.inter * 4);
    L.add("h", slots * d.inter * 4);
    L.add("hq", slots * d.inter);
    L.add("hd", slots * (d.inter / 32) * 4);
    L.add("hs", slots * (d.inter / 32) * 4);
    L.add("out", slots * d.hidden * 4);
    L.add("tbl", (size_t)moe_table_ints(m, d.top_k) * 4);
    // 16-bit activation codes of x and h (qmoe_run_s16)
    L.add("xq16", (size_t)m * d.hidden * 2);
    L.add("hq16", slots * d.inter * 2);
  }
  return L;
}

template <typename T>
T* region(void* ws, const Layout& L, const char* name) {
  bool found = false;
  const size_t off = L.offset(name, &found);
  return found ? reinterpret_cast<T*>(static_cast<char*>(ws) + off) : nullptr;
}

bool fault_injected() {
  const char* e = getenv("QGEMV_FAULT");
  return e && strcmp(e, "launch") == 0;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QGEMV_EHIP, "%s: %s", what, hipGetErrorString(e));
  return QGEMV_OK;
}

int check_gemv_shape(int fmt, int64_t n, int64_t k, const char* what) {
  if (!is_block_fmt(fmt)) return fail(QGEMV_EFORMAT, "%s: format %d is not a block format", what, fmt);
  const int be = fmt_block_elems(fmt);
  if (n < 1 || n > (int64_t)1 << 31) return fail(QGEMV_ESHAPE, "%s: N=%lld out of range", what, (long long)n);
  if (k < be || k % be || k > 65536)
    return fail(QGEMV_ESHAPE, "%s: K=%lld must be a multiple of %d in [%d, 65536]", what, (long long)k, be, be);
  return QGEMV_OK;
}

}  // namespace

extern "C" {

const char* qgemv_status_string(int s) {
  switch (s) {
    case QGEMV_OK: return "ok";
    case QGEMV_EINVAL: return "invalid argument";
    case QGEMV_EFORMAT: return "unsupported format";
    case QGEMV_ESHAPE: return "shape out of range";
    case QGEMV_EALIGN: return "misaligned pointer";
    case QGEMV_EWORKSPACE: return "workspace too small";
    case QGEMV_EVERSION: return "layout version mismatch";
    case QGEMV_EHIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* qgemv_last_error(void) { return g_err; }

int qgemv_create(qgemv_t* out, const qgemv_desc* d) {
  if (!out || !d) return fail(QGEMV_EINVAL, "qgemv_create: null argument");
  *out = nullptr;
  if (d->layout_version != QGEMV_LAYOUT_VERSION)
    return fail(QGEMV_EVERSION, "qgemv_create: layout version %d, library has %d", d->layout_version,
                QGEMV_LAYOUT_VERSION);
  int rc;
  bool need_cb = false;
  switch (d->kind) {
    case QKIND_GEMV:
      if ((rc = check_gemv_shape(d->fmt, d->n, d->k, "gemv")) != QGEMV_OK) return rc;
      if (d->max_m < 1 || d->max_m > 32) return fail(QGEMV_ESHAPE, "gemv: max_m=%d not in 1..32", d->max_m);
      need_cb = has_codebook(d->fmt);
      break;
    case QKIND_FFN:
      if ((rc = check_gemv_shape(d->fmt_gateup, 2 * d->inter, d->hidden, "ffn gate|up")) != QGEMV_OK) return rc;
      if ((rc = check_gemv_shape(d->fmt_down, d->hidden, d->inter, "ffn down")) != QGEMV_OK) return rc;
      if (d->max_m < 1 || d->max_m > kGemvMaxTokens)
        return fail(QGEMV_ESHAPE, "ffn: max_m=%d not in 1..%d", d->max_m, kGemvMaxTokens);
      need_cb = has_codebook(d->fmt_gateup) || has_codebook(d->fmt_down);
      break;
    case QKIND_MOE:
      if (d->n_experts < 1 || d->n_experts > 4096)
        return fail(QGEMV_ESHAPE, "moe: n_experts=%lld not in 1..4096", (long long)d->n_experts);
      if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->n_experts)
        return fail(QGEMV_ESHAPE, "moe: top_k=%d not in 1..min(16, n_experts)", d->top_k);
      if (d->hidden % 32)
        return fail(QGEMV_ESHAPE, "moe: hidden=%lld must be a multiple of 32", (long long)d->hidden);
      if ((rc = check_gemv_shape(d->fmt_expert, 2 * d->inter, d->hidden, "moe gate|up")) != QGEMV_OK) return rc;
      if ((rc = check_gemv_shape(d->fmt_expert, d->hidden, d->inter, "moe down")) != QGEMV_OK) return rc;
      if (d->max_m < 1 || d->max_m > kGemvMaxTokens)
        return fail(QGEMV_ESHAPE, "moe: max_m=%d not in 1..%d", d->max_m, kGemvMaxTokens);
      need_cb = has_codebook(d->fmt_expert);
      break;
    default:
      return fail(QGEMV_EINVAL, "qgemv_create: unknown kind %d", d->kind);
  }
  if (d->kind != QKIND_GEMV && d->inter % 32)
    return fail(QGEMV_ESHAPE, "inter=%lld must be a multiple of 32", (long long)d->inter);
  qgemv_plan* p = new (std::nothrow) qgemv_plan;
  if (!p) return fail(QGEMV_EINVAL, "qgemv_create: out of host memory");
  p->d = *d;
  p->d.codebook16 = nullptr;
  memset(p->cb, 0, sizeof p->cb);
  memset(p->cbw, 0, sizeof p->cbw);
  if (need_cb) {
    if (!d->codebook16) {
      delete p;
      return fail(QGEMV_EINVAL, "IQ4_NL and IQ4_XS need a 16-entry codebook");
    }
    for (int i = 0; i < 16; ++i) p->cb[i] = d->codebook16[i];
    for (int i = 1; i < 16; ++i)
      if (p->cb[i] <= p->cb[i - 1]) {
        delete p;
        return fail(QGEMV_EINVAL, "the codebook must be strictly ascending");
      }
    if (!codebook_pools(p->cb, p->cbw)) {
      delete p;
      return fail(QGEMV_EINVAL, "internal error: codebook pools do not decode");
    }
  }
  *out = p;
  return QGEMV_OK;
}

int qgemv_destroy(qgemv_t h) {
  delete h;
  return QGEMV_OK;
}

int qgemv_workspace_size(qgemv_t h, int m, size_t* bytes) {
  if (!h || !bytes) return fail(QGEMV_EINVAL, "qgemv_workspace_size: null argument");
  if (m < 1 || m > h->d.max_m) return fail(QGEMV_ESHAPE, "m=%d not in 1..%d", m, h->d.max_m);
  *bytes = layout_of(h, m).total();
  return QGEMV_OK;
}

int qgemv_workspace_offset(qgemv_t h, int m, const char* name, size_t* offset) {
  if (!h || !name || !offset) return fail(QGEMV_EINVAL, "qgemv_workspace_offset: null argument");
  if (m < 1 || m > h->d.max_m) return fail(QGEMV_ESHAPE, "m=%d not in 1..%d", m, h->d.max_m);
  bool found = false;
  *offset = layout_of(h, m).offset(name, &found);
  if (!found) return fail(QGEMV_EINVAL, "workspace has no region '%s'", name);
  return QGEMV_OK;
}

int qgemv_weight_bytes(qgemv_t h, int which, size_t* bytes) {
  if (!h || !bytes) return fail(QGEMV_EINVAL, "qgemv_weight_bytes: null argument");
  const qgemv_desc& d = h->d;
  size_t b = 0;
  if (d.kind == QKIND_GEMV && which == 0) b = (size_t)d.n * fmt_row_bytes(d.fmt, d.k);
  else if (d.kind == QKIND_FFN && which == 0) b = (size_t)2 * d.inter * fmt_row_bytes(d.fmt_gateup, d.hidden);
  else if (d.kind == QKIND_FFN && which == 1) b = (size_t)d.hidden * fmt_row_bytes(d.fmt_down, d.inter);
  else if (d.kind == QKIND_MOE && (which == 0 || which == 2))
    b = (size_t)(which == 0 ? d.n_experts : 1) * 2 * d.inter * fmt_row_bytes(d.fmt_expert, d.hidden);
  else if (d.kind == QKIND_MOE && (which == 1 || which == 3))
    b = (size_t)(which == 1 ? d.n_experts : 1) * d.hidden * fmt_row_bytes(d.fmt_expert, d.inter);
  else if (d.kind == QKIND_MOE && which == 4) b = (size_t)d.n_experts * d.hidden * 4;
  else return fail(QGEMV_EINVAL, "weight buffer %d does not exist for this plan", which);
  *bytes = round_up(b, 16);
  return QGEMV_OK;
}

namespace {

// Largest K for which qgemv_run fuses the activation quantizer into the GEMV.
#ifndef QG_FUSED_MAXK
#define QG_FUSED_MAXK 4096
#endif
constexpr int64_t kFusedQuantMaxK = QG_FUSED_MAXK;

// Whether the GEMV kernel quantizes x itself (one launch) rather than after
// a separate quantizer launch. Every workgroup of a fused launch quantizes
// all of x, which pays for the saved launch only for one token. Measured on
// MI355X (qgemv_run, weights from HBM): one token, K = 2048: 1.0-1.2 us
// faster for Q4_0, Q8_0 and Q4_K; K = 4096: 1.0 us faster for Q8_0 at 4096
// rows, even for Q8_0 / Q4_K / Q4_0 / Q6_K at 12288 rows; Q5_K and IQ4_XS
// (register-direct kernel) 4096 -> 12288: 11.6 -> 9.8 and 9.5 -> 7.5 us; but
// slower for the LDS-staged IQ4_NL (the lm_head 4096 -> 248320: 101.8
// against 97.7 us sustained); four or sixteen tokens: 1-15 us slower for
// every format.
bool fuse_quantizer(int fmt, int64_t k, int m) {
  if (m != 1 || k > kFusedQuantMaxK) return false;
  return k <= 2048 || fmt == kQ4_0 || fmt == kQ8_0 || fmt == kQ4_K || fmt == kQ6_K || fmt == kIQ4_XS || fmt == kQ5_K;
}

int validate_gemv_call(qgemv_t h, int m, const void* ws, size_t ws_bytes, const char* fn) {
  if (!h || h->d.kind != QKIND_GEMV) return fail(QGEMV_EINVAL, "%s: not a GEMV plan", fn);
  if (!ws) return fail(QGEMV_EINVAL, "%s: null workspace", fn);
  if (!aligned(ws, 256)) return fail(QGEMV_EALIGN, "%s: ws needs 256-byte alignment", fn);
  if (m < 1 || m > h->d.max_m) return fail(QGEMV_ESHAPE, "%s: m=%d not in 1..%d", fn, m, h->d.max_m);
  const size_t need = layout_of(h, m).total();
  if (ws_bytes < need) return fail(QGEMV_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  return QGEMV_OK;
}

int gemv_quantize(qgemv_t h, const float* x, int m, void* ws, hipStream_t s) {
  const Layout L = layout_of(h, m);
  TiledAct t;
  if (m >= kMfmaMinTokens) {
    t.codes = region<int8_t>(ws, L, "xqt");
    t.dx = region<float>(ws, L, "dxt");
    t.c = region<float>(ws, L, "cxt");
    t.kblocks = (int)(h->d.k / 32);
  }
  return check_launch(launch_quant_q8(x, region<int8_t>(ws, L, "xq"), region<float>(ws, L, "dx"),
                                      region<int32_t>(ws, L, "sx"), (int64_t)m * (h->d.k / 32), s,
                                      m >= kMfmaMinTokens ? &t : nullptr),
                      "quantize");
}

int gemv_from_quantized(qgemv_t h, const void* w, float* y, int m, const void* ws, hipStream_t s) {
  const qgemv_desc& d = h->d;
  const Layout L = layout_of(h, m);
  void* wsm = const_cast<void*>(ws);
  const int8_t* xq = region<int8_t>(wsm, L, "xq");
  const float* dx = region<float>(wsm, L, "dx");
  const int32_t* sx = region<int32_t>(wsm, L, "sx");
  if (m >= kMfmaMinTokens && mfma_supported(d.fmt)) {
    return check_launch(launch_gemm32(d.fmt, static_cast<const uint8_t*>(w), region<int8_t>(wsm, L, "xqt"),
                                      region<float>(wsm, L, "dxt"), region<float>(wsm, L, "cxt"), y, d.n, d.k, m, s),
                        "gemm32");
  }
  GemvProblem p;
  p.w = static_cast<const uint8_t*>(w);
  p.xq = xq;
  p.dx = dx;
  p.xs = d.k;
  p.y = y;
  p.ldy = d.n;
  p.n = d.n;
  p.k = d.k;
  memcpy(p.cb, h->cbw, sizeof p.cb);
  for (int t0 = 0; t0 < m; t0 += kGemvMaxTokens) {
    GemvProblem c = p;
    c.m = (m - t0) < kGemvMaxTokens ? (m - t0) : kGemvMaxTokens;
    c.xq = xq + (int64_t)t0 * d.k;
    c.dx = dx + (int64_t)t0 * (d.k / 32);
    c.y = y + (int64_t)t0 * d.n;
    int rc = check_launch(launch_gemv(d.fmt, c, false, s), "gemv");
    if (rc) return rc;
  }
  return QGEMV_OK;
}

}  // namespace

namespace {

// qgemv_run after validation: the workspace `ws` holds at least
// layout_of(h, m).total() bytes.
int gemv_run(qgemv_t h, const void* w, const float* x, float* y, int m, void* ws, hipStream_t s) {
  int rc;
  const qgemv_desc& d = h->d;
  if (m > kGemvMaxTokens || !fuse_quantizer(d.fmt, d.k, m) || (m >= kMfmaMinTokens && mfma_supported(d.fmt))) {
    if ((rc = gemv_quantize(h, x, m, ws, s))) return rc;
    return gemv_from_quantized(h, w, y, m, ws, s);
  }
  // One token, short rows: one launch, the GEMV kernel quantizes x in its
  // prologue (same arithmetic as the standalone quantizer) and its first
  // workgroup stores the codes in the workspace regions "xq", "dx", "sx".
  const Layout L = layout_of(h, m);
  GemvProblem p;
  p.w = static_cast<const uint8_t*>(w);
  p.xf = x;
  p.xs = d.k;
  p.xq_out = region<int8_t>(ws, L, "xq");
  p.dx_out = region<float>(ws, L, "dx");
  p.sx_out = region<int32_t>(ws, L, "sx");
  p.y = y;
  p.ldy = d.n;
  p.n = d.n;
  p.k = d.k;
  p.m = m;
  memcpy(p.cb, h->cbw, sizeof p.cb);
  return check_launch(launch_gemv(d.fmt, p, false, s), "gemv");
}

}  // namespace

int qgemv_run(qgemv_t h, const void* w, const float* x, float* y, int m, void* ws, size_t ws_bytes,
              void* stream) {
  int rc = validate_gemv_call(h, m, ws, ws_bytes, "qgemv_run");
  if (rc) return rc;
  if (!w || !x || !y) return fail(QGEMV_EINVAL, "qgemv_run: null pointer");
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4))
    return fail(QGEMV_EALIGN, "qgemv_run: w and x need 16-byte, y 4-byte alignment");
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_run: launch failure injected (QGEMV_FAULT)");
  return gemv_run(h, w, x, y, m, ws, static_cast<hipStream_t>(stream));
}

int qgemv_run_noalloc(qgemv_t h, const void* w, const float* x, float* y, int m, void* stream) {
  if (!h || h->d.kind != QKIND_GEMV) return fail(QGEMV_EINVAL, "qgemv_run_noalloc: not a GEMV plan");
  if (m < 1 || m > h->d.max_m) return fail(QGEMV_ESHAPE, "qgemv_run_noalloc: m=%d not in 1..%d", m, h->d.max_m);
  if (!w || !x || !y) return fail(QGEMV_EINVAL, "qgemv_run_noalloc: null pointer");
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4))
    return fail(QGEMV_EALIGN, "qgemv_run_noalloc: w and x need 16-byte, y 4-byte alignment");
  const size_t need = layout_of(h, m).total();
  if (need > kNoAllocScratchBytes)
    return fail(QGEMV_EWORKSPACE,
                "qgemv_run_noalloc: this call needs %zu bytes of workspace, more than the fixed %zu-byte device "
                "scratch; use qgemv_run with a caller-allocated workspace",
                need, kNoAllocScratchBytes);
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_run_noalloc: launch failure injected (QGEMV_FAULT)");
  void* ws = nullptr;
  int rc = check_launch(noalloc_scratch(&ws), "qgemv_run_noalloc: device scratch");
  if (rc) return rc;
  return gemv_run(h, w, x, y, m, ws, static_cast<hipStream_t>(stream));
}

int qgemv_quantize(qgemv_t h, const float* x, int m, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_gemv_call(h, m, ws, ws_bytes, "qgemv_quantize");
  if (rc) return rc;
  if (!x) return fail(QGEMV_EINVAL, "qgemv_quantize: null pointer");
  if (!aligned(x, 16)) return fail(QGEMV_EALIGN, "qgemv_quantize: x needs 16-byte alignment");
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_quantize: launch failure injected (QGEMV_FAULT)");
  return gemv_quantize(h, x, m, ws, static_cast<hipStream_t>(stream));
}

int qgemv_run_quantized(qgemv_t h, const void* w, float* y, int m, const void* ws, size_t ws_bytes,
                        void* stream) {
  int rc = validate_gemv_call(h, m, ws, ws_bytes, "qgemv_run_quantized");
  if (rc) return rc;
  if (!w || !y) return fail(QGEMV_EINVAL, "qgemv_run_quantized: null pointer");
  if (!aligned(w, 16) || !aligned(y, 4))
    return fail(QGEMV_EALIGN, "qgemv_run_quantized: w needs 16-byte, y 4-byte alignment");
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_run_quantized: launch failure injected (QGEMV_FAULT)");
  return gemv_from_quantized(h, w, y, m, ws, static_cast<hipStream_t>(stream));
}

int qffn_run(qgemv_t h, const void* w_gateup, const void* w_down, const float* x, float* y, int m,
             void* ws, size_t ws_bytes, void* stream) {
  if (!h || h->d.kind != QKIND_FFN) return fail(QGEMV_EINVAL, "qffn_run: not an FFN plan");
  if (!w_gateup || !w_down || !x || !y || !ws) return fail(QGEMV_EINVAL, "qffn_run: null pointer");
  if (!aligned(w_gateup, 16) || !aligned(w_down, 16) || !aligned(x, 16) || !aligned(y, 4) ||
      !aligned(ws, 256))
    return fail(QGEMV_EALIGN, "qffn_run: weights and x need 16-byte, y 4-byte, ws 256-byte alignment");
  const qgemv_desc& d = h->d;
  if (m < 1 || m > d.max_m) return fail(QGEMV_ESHAPE, "qffn_run: m=%d not in 1..%d", m, d.max_m);
  const Layout L = layout_of(h, m);
  if (ws_bytes < L.total())
    return fail(QGEMV_EWORKSPACE, "qffn_run: workspace %zu < %zu bytes", ws_bytes, L.total());
  if (fault_injected()) return fail(QGEMV_EHIP, "qffn_run: launch failure injected (QGEMV_FAULT)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int8_t* xq = region<int8_t>(ws, L, "xq");
  float* dx = region<float>(ws, L, "dx");
  int32_t* sx = region<int32_t>(ws, L, "sx");
  float* gu = region<float>(ws, L, "gu");
  float* hh = region<float>(ws, L, "h");
  int8_t* hq = region<int8_t>(ws, L, "hq");
  float* hd = region<float>(ws, L, "hd");
  int32_t* hs = region<int32_t>(ws, L, "hs");
  int rc;
  GemvProblem p;
  p.w = static_cast<const uint8_t*>(w_gateup);
  if (fuse_quantizer(d.fmt_gateup, d.hidden, m)) {
    p.xf = x;  // quantized in the gate|up kernel's prologue, codes stored in ws
    p.xq_out = xq;
    p.dx_out = dx;
    p.sx_out = sx;
  } else {
    // Several tokens or long rows: one quantizer launch is cheaper than
    // every workgroup of the gate|up GEMV quantizing x again.
    if ((rc = check_launch(launch_quant_q8(x, xq, dx, sx, (int64_t)m * d.hidden / 32, s), "quantize"))) return rc;
    p.xq = xq;
    p.dx = dx;
  }
  p.xs = d.hidden;
  p.y = gu;
  p.ldy = 2 * d.inter;
  p.n = 2 * d.inter;
  p.k = d.hidden;
  p.m = m;
  memcpy(p.cb, h->cbw, sizeof p.cb);
  if ((rc = check_launch(launch_gemv(d.fmt_gateup, p, false, s), "gate|up gemv"))) return rc;
  if ((rc = check_launch(launch_swiglu_q8(gu, 2 * d.inter, hh, hq, hd, hs, m, d.inter, s), "swiglu")))
    return rc;
  GemvProblem q = p;
  q.xf = nullptr;
  q.xq_out = nullptr;
  q.dx_out = nullptr;
  q.sx_out = nullptr;
  q.w = static_cast<const uint8_t*>(w_down);
  q.xq = hq;
  q.dx = hd;
  q.xs = d.inter;
  q.y = y;
  q.ldy = d.hidden;
  q.n = d.hidden;
  q.k = d.inter;
  return check_launch(launch_gemv(d.fmt_down, q, false, s), "down gemv");
}

namespace {
int moe_run(qgemv_t h, const float* w_router, const void* w_experts_gateup, const void* w_experts_down,
            const void* w_shared_gateup, const void* w_shared_down, const float* x, float* y, int m, void* ws,
            size_t ws_bytes, void* stream, bool s16, const char* fn) {
  if (!h || h->d.kind != QKIND_MOE) return fail(QGEMV_EINVAL, "%s: not a MoE plan", fn);
  if (!w_router || !w_experts_gateup || !w_experts_down || !w_shared_gateup || !w_shared_down || !x ||
      !y || !ws)
    return fail(QGEMV_EINVAL, "%s: null pointer", fn);
  if (!aligned(w_router, 16) || !aligned(w_experts_gateup, 16) || !aligned(w_experts_down, 16) ||
      !aligned(w_shared_gateup, 16) || !aligned(w_shared_down, 16) || !aligned(x, 16) ||
      !aligned(y, 4) || !aligned(ws, 256))
    return fail(QGEMV_EALIGN, "%s: weights and x need 16-byte, y 4-byte, ws 256-byte alignment", fn);
  const qgemv_desc& d = h->d;
  if (m < 1 || m > d.max_m) return fail(QGEMV_ESHAPE, "%s: m=%d not in 1..%d", fn, m, d.max_m);
  const int64_t gu_bytes = 2 * d.inter * fmt_row_bytes(d.fmt_expert, d.hidden);
  const int64_t dn_bytes = d.hidden * fmt_row_bytes(d.fmt_expert, d.inter);
  if (gu_bytes % 16 || dn_bytes % 16)
    return fail(QGEMV_ESHAPE, "%s: expert matrices must be multiples of 16 bytes", fn);
  if (s16 && d.fmt_expert != QFMT_Q4_0)
    return fail(QGEMV_EFORMAT, "%s: 16-bit activations need Q4_0 experts", fn);
  if (s16 && (!q40_s16_grouped_ok(d.hidden) || !q40_s16_grouped_ok(d.inter)))
    return fail(QGEMV_ESHAPE, "%s: 16-bit experts need hidden and inter in {512, 1024, 2048, 4096}", fn);
  const Layout L = layout_of(h, m);
  if (ws_bytes < L.total())
    return fail(QGEMV_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, L.total());
  if (fault_injected()) return fail(QGEMV_EHIP, "%s: launch failure injected (QGEMV_FAULT)", fn);
  MoeCall c;
  c.router = w_router;
  c.gu = static_cast<const uint8_t*>(w_experts_gateup);
  c.dn = static_cast<const uint8_t*>(w_experts_down);
  c.gu_shared = static_cast<const uint8_t*>(w_shared_gateup);
  c.dn_shared = static_cast<const uint8_t*>(w_shared_down);
  c.gu_stride = gu_bytes;
  c.dn_stride = dn_bytes;
  c.x = x;
  c.y = y;
  c.m = m;
  c.hidden = d.hidden;
  c.inter = d.inter;
  c.n_experts = (int)d.n_experts;
  c.top_k = d.top_k;
  c.fmt = d.fmt_expert;
  memcpy(c.cb, h->cbw, sizeof c.cb);
  c.logits = region<float>(ws, L, "logits");
  c.ids = region<int32_t>(ws, L, "ids");
  c.wts = region<float>(ws, L, "wts");
  c.xq = region<int8_t>(ws, L, "xq");
  c.dx = region<float>(ws, L, "dx");
  c.sx = region<int32_t>(ws, L, "sx");
  c.gu_out = region<float>(ws, L, "gu");
  c.h = region<float>(ws, L, "h");
  c.hq = region<int8_t>(ws, L, "hq");
  c.hd = region<float>(ws, L, "hd");
  c.hs = region<int32_t>(ws, L, "hs");
  c.out = region<float>(ws, L, "out");
  c.tbl = region<int32_t>(ws, L, "tbl");
  if (s16) {
    c.xq16 = region<int16_t>(ws, L, "xq16");
    c.hq16 = region<int16_t>(ws, L, "hq16");
  }
  return check_launch(launch_moe(c, static_cast<hipStream_t>(stream)), "moe");
}
}  // namespace

int qmoe_run(qgemv_t h, const float* w_router, const void* w_experts_gateup, const void* w_experts_down,
             const void* w_shared_gateup, const void* w_shared_down, const float* x, float* y, int m,
             void* ws, size_t ws_bytes, void* stream) {
  return moe_run(h, w_router, w_experts_gateup, w_experts_down, w_shared_gateup, w_shared_down, x, y, m, ws,
                 ws_bytes, stream, false, "qmoe_run");
}

int qmoe_run_s16(qgemv_t h, const float* w_router, const void* w_experts_gateup, const void* w_experts_down,
                 const void* w_shared_gateup, const void* w_shared_down, const float* x, float* y, int m,
                 void* ws, size_t ws_bytes, void* stream) {
  return moe_run(h, w_router, w_experts_gateup, w_experts_down, w_shared_gateup, w_shared_down, x, y, m, ws,
                 ws_bytes, stream, true, "qmoe_run_s16");
}

int qgemv_debug_quantize(const float* x, int8_t* xq, float* dx, int32_t* sx, int m, int64_t k, void* stream) {
  if (!x || !xq || !dx || !sx) return fail(QGEMV_EINVAL, "qgemv_debug_quantize: null pointer");
  if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(dx, 4) || !aligned(sx, 4))
    return fail(QGEMV_EALIGN, "qgemv_debug_quantize: x needs 16-byte, outputs 4-byte alignment");
  if (m < 1 || k < 32 || k % 32) return fail(QGEMV_ESHAPE, "qgemv_debug_quantize: bad m/k");
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_debug_quantize: launch failure injected");
  return check_launch(launch_quant_q8(x, xq, dx, sx, (int64_t)m * (k / 32), static_cast<hipStream_t>(stream)),
                      "quantize");
}

int qgemv_debug_block_dots(qgemv_t h, const void* w, const int8_t* xq, int32_t* dots, int m, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!h || h->d.kind != QKIND_GEMV) return fail(QGEMV_EINVAL, "qgemv_debug_block_dots: not a GEMV plan");
  if (!w || !xq || !dots) return fail(QGEMV_EINVAL, "qgemv_debug_block_dots: null pointer");
  if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(dots, 4))
    return fail(QGEMV_EALIGN, "qgemv_debug_block_dots: w and xq need 16-byte alignment");
  const qgemv_desc& d = h->d;
  if (m < 1 || m > d.max_m) return fail(QGEMV_ESHAPE, "qgemv_debug_block_dots: m=%d not in 1..%d", m, d.max_m);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m >= kMfmaMinTokens && mfma_supported(d.fmt)) {
    // The batched path reads the token-tiled codes from the workspace.
    int rc = validate_gemv_call(h, m, ws, ws_bytes, "qgemv_debug_block_dots");
    if (rc) return rc;
    if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_debug_block_dots: launch failure injected");
    const Layout L = layout_of(h, m);
    int8_t* xqt = region<int8_t>(ws, L, "xqt");
    if ((rc = check_launch(launch_tile_codes(xq, xqt, m, (int)(d.k / 32), s), "tile codes"))) return rc;
    return check_launch(launch_gemm32_dots(d.fmt, static_cast<const uint8_t*>(w), xqt, dots, d.n, d.k, m, s),
                        "gemm32 dots");
  }
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_debug_block_dots: launch failure injected");
  GemvProblem p;
  p.w = static_cast<const uint8_t*>(w);
  p.xq = xq;
  p.dx = nullptr;  // the integer epilogue never reads scales
  p.xs = d.k;
  p.dots = dots;
  p.n = d.n;
  p.k = d.k;
  memcpy(p.cb, h->cbw, sizeof p.cb);
  const int64_t per_tok = d.n * (d.k / (d.fmt == QFMT_Q6_K ? 16 : 32));
  for (int t0 = 0; t0 < m; t0 += kGemvMaxTokens) {
    GemvProblem c = p;
    c.m = (m - t0) < kGemvMaxTokens ? (m - t0) : kGemvMaxTokens;
    c.xq = xq + (int64_t)t0 * d.k;
    c.dots = dots + (int64_t)t0 * per_tok;
    int rc = check_launch(launch_gemv(d.fmt, c, true, s), "block dots");
    if (rc) return rc;
  }
  return QGEMV_OK;
}

namespace {
int attn_shape(int n_heads, int n_kv_heads, int head_dim, int64_t n_ctx, AttnShape& a, const char* fn) {
  a.n_heads = n_heads;
  a.n_kv = n_kv_heads;
  a.head_dim = head_dim;
  a.n_ctx = n_ctx;
  if (!attn_supported(a))
    return fail(QGEMV_ESHAPE,
                "%s: unsupported shape heads=%d kv_heads=%d head_dim=%d n_ctx=%lld (head_dim 128/256, "
                "heads/kv_heads in {1,2,4,8}, 1 <= n_ctx, n_ctx*head_dim*2 + 4096 < 2^31)",
                fn, n_heads, n_kv_heads, head_dim, (long long)n_ctx);
  return QGEMV_OK;
}
}  // namespace

int qattn_workspace_size(int n_heads, int n_kv_heads, int head_dim, int64_t n_ctx, size_t* bytes) {
  if (!bytes) return fail(QGEMV_EINVAL, "qattn_workspace_size: null pointer");
  AttnShape a;
  int rc = attn_shape(n_heads, n_kv_heads, head_dim, n_ctx, a, "qattn_workspace_size");
  if (rc) return rc;
  *bytes = attn_workspace_bytes(a);
  return QGEMV_OK;
}

int qattn_decode(const float* q, const void* k_cache, const void* v_cache, float* out, int n_heads,
                 int n_kv_heads, int head_dim, int64_t n_ctx, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !out) return fail(QGEMV_EINVAL, "qattn_decode: null pointer");
  AttnShape a;
  int rc = attn_shape(n_heads, n_kv_heads, head_dim, n_ctx, a, "qattn_decode");
  if (rc) return rc;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(QGEMV_EALIGN, "qattn_decode: q, caches and out need 16-byte alignment");
  const size_t need = attn_workspace_bytes(a);
  if (need) {
    if (!ws) return fail(QGEMV_EINVAL, "qattn_decode: this context needs a workspace of %zu bytes", need);
    if (!aligned(ws, 256)) return fail(QGEMV_EALIGN, "qattn_decode: ws needs 256-byte alignment");
    if (ws_bytes < need) return fail(QGEMV_EWORKSPACE, "qattn_decode: workspace %zu < %zu bytes", ws_bytes, need);
  }
  if (fault_injected()) return fail(QGEMV_EHIP, "qattn_decode: launch failure injected (QGEMV_FAULT)");
  return check_launch(launch_attn(a, q, static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                                  out, ws, static_cast<hipStream_t>(stream)),
                      "attention");
}

namespace {
int s16_plan(qgemv_t h, const char* fn) {
  if (!h || h->d.kind != QKIND_GEMV) return fail(QGEMV_EINVAL, "%s: not a GEMV plan", fn);
  if (h->d.fmt != QFMT_Q4_K && h->d.fmt != QFMT_Q5_K)
    return fail(QGEMV_EFORMAT, "%s: 16-bit activations need a Q4_K or Q5_K plan", fn);
  if (!s16_gemv_ok(h->d.fmt, h->d.n, h->d.k))
    return fail(QGEMV_ESHAPE, "%s: k=%lld must be a multiple of 2048 up to 8192", fn, (long long)h->d.k);
  return QGEMV_OK;
}
size_t s16_ws_bytes(int64_t k) { return round_up((size_t)k * 2, 256) + 2 * round_up((size_t)(k / 32) * 4, 256); }
}  // namespace

int qgemv_workspace_size_s16(qgemv_t h, size_t* bytes) {
  int rc = s16_plan(h, "qgemv_workspace_size_s16");
  if (rc) return rc;
  if (!bytes) return fail(QGEMV_EINVAL, "qgemv_workspace_size_s16: null pointer");
  *bytes = s16_ws_bytes(h->d.k);
  return QGEMV_OK;
}

int qgemv_run_s16(qgemv_t h, const void* w, const float* x, float* y, void* ws, size_t ws_bytes, void* stream) {
  int rc = s16_plan(h, "qgemv_run_s16");
  if (rc) return rc;
  if (!w || !x || !y || !ws) return fail(QGEMV_EINVAL, "qgemv_run_s16: null pointer");
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(ws, 256))
    return fail(QGEMV_EALIGN, "qgemv_run_s16: w and x need 16-byte, y 4-byte, ws 256-byte alignment");
  const int64_t k = h->d.k;
  if (ws_bytes < s16_ws_bytes(k))
    return fail(QGEMV_EWORKSPACE, "qgemv_run_s16: workspace %zu < %zu bytes", ws_bytes, s16_ws_bytes(k));
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_run_s16: launch failure injected (QGEMV_FAULT)");
  char* base = static_cast<char*>(ws);
  int16_t* xq = reinterpret_cast<int16_t*>(base);
  float* dx = reinterpret_cast<float*>(base + round_up((size_t)k * 2, 256));
  int32_t* sx = reinterpret_cast<int32_t*>(base + round_up((size_t)k * 2, 256) + round_up((size_t)(k / 32) * 4, 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((rc = check_launch(launch_quant_s16(x, xq, dx, sx, k / 32, s), "quantize s16"))) return rc;
  return check_launch(
      launch_kquant_s16(h->d.fmt, static_cast<const uint8_t*>(w), xq, dx, sx, y, nullptr, h->d.n, k, s),
      "gemv s16");
}

int qgemv_run_f32act(qgemv_t h, const void* w, const float* x, float* y, int m, void* stream) {
  if (!h || h->d.kind != QKIND_GEMV) return fail(QGEMV_EINVAL, "qgemv_run_f32act: not a GEMV plan");
  if (!fact_supported(h->d.fmt))
    return fail(QGEMV_EFORMAT, "qgemv_run_f32act: float activations need a Q4_0 or Q8_0 plan");
  if (m < 1 || m > 32) return fail(QGEMV_ESHAPE, "qgemv_run_f32act: m=%d not in 1..32", m);
  if (!w || !x || !y) return fail(QGEMV_EINVAL, "qgemv_run_f32act: null pointer");
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4))
    return fail(QGEMV_EALIGN, "qgemv_run_f32act: w and x need 16-byte, y 4-byte alignment");
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_run_f32act: launch failure injected (QGEMV_FAULT)");
  return check_launch(launch_fact(h->d.fmt, static_cast<const uint8_t*>(w), x, y, m, h->d.n, h->d.k,
                                  static_cast<hipStream_t>(stream)),
                      "gemv f32act");
}

int qgemv_debug_quantize_s16(const float* x, int16_t* xq, float* dx, int32_t* sx, int m, int64_t k, void* stream) {
  if (!x || !xq || !dx || !sx) return fail(QGEMV_EINVAL, "qgemv_debug_quantize_s16: null pointer");
  if (!aligned(x, 16) || !aligned(xq, 8) || !aligned(dx, 4) || !aligned(sx, 4))
    return fail(QGEMV_EALIGN, "qgemv_debug_quantize_s16: x needs 16-byte, xq 8-byte, others 4-byte alignment");
  if (m < 1 || k < 32 || k % 32) return fail(QGEMV_ESHAPE, "qgemv_debug_quantize_s16: bad m/k");
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_debug_quantize_s16: launch failure injected");
  return check_launch(launch_quant_s16(x, xq, dx, sx, (int64_t)m * (k / 32), static_cast<hipStream_t>(stream)),
                      "quantize s16");
}

int qgemv_debug_block_dots_s16(qgemv_t h, const void* w, const int16_t* xq, int32_t* dots, void* stream) {
  int rc = s16_plan(h, "qgemv_debug_block_dots_s16");
  if (rc) return rc;
  if (!w || !xq || !dots) return fail(QGEMV_EINVAL, "qgemv_debug_block_dots_s16: null pointer");
  if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(dots, 4))
    return fail(QGEMV_EALIGN, "qgemv_debug_block_dots_s16: w and xq need 16-byte alignment");
  if (fault_injected()) return fail(QGEMV_EHIP, "qgemv_debug_block_dots_s16: launch failure injected");
  return check_launch(launch_kquant_s16(h->d.fmt, static_cast<const uint8_t*>(w), xq, nullptr, nullptr, nullptr,
                                        dots, h->d.n, h->d.k, static_cast<hipStream_t>(stream)),
                      "block dots s16");
}

int qgemv_debug_clear_launch_cache(void) {
  clear_launch_cache();
  return QGEMV_OK;
}

int qgemv_debug_stream_read(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out) return fail(QGEMV_EINVAL, "qgemv_debug_stream_read: null pointer");
  if (!aligned(buf, 16) || !aligned(out, 4) || bytes % 16)
    return fail(QGEMV_EALIGN, "qgemv_debug_stream_read: buf and bytes need 16-byte alignment");
  return check_launch(launch_stream_read(buf, bytes, out, static_cast<hipStream_t>(stream)), "stream read");
}

}  // extern "C"
