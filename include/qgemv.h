/*
 * qgemv.h -- C ABI of the block-quantized decode GEMV library for AMD MI355X
 * (gfx950).
 *
 * The library multiplies fp32 activations by weights that stay in their
 * packed block-quantized form in device memory (no fp16 or int8 expansion of
 * the matrix). Activations are quantized on the device into 32-element int8
 * blocks with one fp32 scale; each weight block is decoded in registers and
 * combined with the activations by int8 dot products, then scaled (with the
 * min correction of the K-quant super-blocks, or a 16-entry codebook for the
 * non-linear 4-bit format). This is the in-place GEMV over GGUF-style blocks
 * described in "Why expert caching can't save dense models: running a 27B
 * dense model in 16 GB VRAM" (xhh.club; section on in-place quantized compute
 * and single-stream fusion, and its Q&A on computing GGUF blocks without
 * FP16 expansion).
 *
 * Boundary style: a pure C ABI, loadable at run time, whose functions return
 * a status code and never abort -- the convention of the standalone device
 * module in "01 · Phase overview: from 2B to 8B to MoE" (icman.com.cn,
 * section 一 and ledger item ①: a pure-C module boundary with a 0-on-success
 * device layer). Unlike that module there is no CPU fallback: a call either
 * runs on the GPU or returns an error.
 *
 * Conventions for every entry point:
 *  - Return 0 (QGEMV_OK) on success, a negative QGEMV_E* code on error.
 *    Argument validation is done on the host before anything is enqueued; a
 *    failed call enqueues nothing. qgemv_last_error() gives a per-thread
 *    message for the last failure.
 *  - Pointers named w*, x, y, ws, dots, w_router are DEVICE pointers owned by
 *    the caller (for example torch tensors' data_ptr()). The library never
 *    allocates or frees device memory and never synchronizes; it only
 *    enqueues kernels on the caller's stream (`stream` is a hipStream_t; NULL
 *    is the default stream). Asynchronous device faults surface at the
 *    caller's next synchronization.
 *  - Handles (qgemv_t) are immutable host-side plans that own only host
 *    memory. One handle may be used concurrently from several threads and
 *    streams, provided each concurrent call has its own workspace and output.
 *    The launch facts the library caches (compute units per device, resident
 *    workgroups per kernel, raised LDS limits) are kept per device and filled
 *    under a lock, so first calls from several threads, on several devices
 *    or inside stream capture are safe.
 *  - Layouts are row-major. A weight matrix with N rows and K inputs is N
 *    rows of (K / block_elems) blocks, block_bytes each, rows contiguous,
 *    starting at a 16-byte aligned address. The buffer must be readable up to
 *    the next 16-byte boundary after its last block (128-bit loads may touch
 *    those pad bytes, whose contents are ignored): allocate at least
 *    qgemv_weight_bytes() bytes.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version of the block byte layouts below. A plan created with another
 * version is refused, so packed weights and library always move together. */
#define QGEMV_LAYOUT_VERSION 1

/* Status codes. */
enum {
  QGEMV_OK = 0,
  QGEMV_EINVAL = -1,     /* null pointer, bad kind, bad handle, bad enum   */
  QGEMV_EFORMAT = -2,    /* format not supported for this kind / path      */
  QGEMV_ESHAPE = -3,     /* N, K, M or expert shape out of range           */
  QGEMV_EALIGN = -4,     /* pointer misaligned (weights need 16 B)         */
  QGEMV_EWORKSPACE = -5, /* workspace too small                            */
  QGEMV_EVERSION = -6,   /* layout_version != QGEMV_LAYOUT_VERSION         */
  QGEMV_EHIP = -7        /* the HIP runtime refused a launch               */
};

/* Weight formats. Byte layouts (little-endian, fp16 = IEEE binary16):
 *  QFMT_F32    fp32 matrix (router only).
 *  QFMT_Q4_0   32 elements / 18 B: d fp16 | qs[16]. Element i < 16 is the low
 *              nibble of qs[i], element i >= 16 the high nibble of qs[i-16].
 *              value = d * (q - 8).
 *  QFMT_Q8_0   32 elements / 34 B: d fp16 | 32 int8 codes. value = d * q.
 *  QFMT_Q4_K   256 elements / 144 B: d fp16 | dmin fp16 | scales[12] |
 *              qs[128]. scales is a 96-bit little-endian stream of sixteen
 *              6-bit fields (field f at bits 6f..6f+5): sc_0..sc_7 then
 *              m_0..m_7. Sub-block j (32 elements) has its codes in
 *              qs[16j..16j+15] in the Q4_0 nibble order.
 *              value = d * sc_j * q - dmin * m_j.
 *  QFMT_Q6_K   256 elements / 210 B: d fp16 | sc[16] int8 | ql[128] |
 *              qh[64]. Element 32g + i: low 4 bits in ql[16g + i % 16] (low
 *              nibble if i < 16, else high), high 2 bits at bits
 *              2*(i / 8)..+1 of qh[8g + i % 8]. Sub-block j = element / 16.
 *              value = d * sc_j * (q - 32).
 *  QFMT_IQ4_NL 32 elements / 18 B: Q4_0 layout; value = d * codebook[q],
 *              codebook = 16 sorted int8 given at plan creation.
 *  QFMT_Q5_K   256 elements / 176 B: d fp16 | dmin fp16 | scales[12] (as
 *              Q4_K) | qh[32] | qs[128] (low 4 bits, as Q4_K). The fifth
 *              bit of element 32j + i is bit i / 4 of qh[4j + i % 4].
 *              q = low | fifth << 4 (0..31); value = d * sc_j * q - dmin * m_j.
 *  QFMT_IQ4_XS 256 elements / 136 B: d fp16 | scales_h u16 | scales_l[4] |
 *              qs[128] (4-bit indices, as Q4_K). Sub-scale ls_j (0..63) =
 *              nibble j % 2 of scales_l[j / 2] (low nibble first) | bits
 *              2j..2j+1 of scales_h as bits 4..5.
 *              value = d * (ls_j - 32) * codebook[q].
 * The per-format value formulas are those of the decode-GEMV workloads the
 * library targets (Q5_K and IQ4_XS: the formats whose single-matrix
 * bandwidth the pages report); the pages give no byte order, so the order
 * above is this library's own and is versioned by QGEMV_LAYOUT_VERSION. */
enum {
  QFMT_F32 = 0,
  QFMT_Q4_0 = 1,
  QFMT_Q8_0 = 2,
  QFMT_Q4_K = 3,
  QFMT_Q6_K = 4,
  QFMT_IQ4_NL = 5,
  QFMT_Q5_K = 6,
  QFMT_IQ4_XS = 7
};

enum { QKIND_GEMV = 0, QKIND_FFN = 1, QKIND_MOE = 2 };

/* Plan descriptor. Unused fields must be zero. */
typedef struct qgemv_desc {
  int32_t kind;            /* QKIND_*                                        */
  int32_t layout_version;  /* must be QGEMV_LAYOUT_VERSION                   */
  /* QKIND_GEMV: y[m, n] = W[n, k] . x[m, k]                                 */
  int32_t fmt;             /* QFMT_Q4_0 .. QFMT_IQ4_XS                       */
  int32_t max_m;           /* largest m passed to qgemv_run (1..32)          */
  int64_t n;               /* rows (outputs), >= 1                           */
  int64_t k;               /* inputs, multiple of the format's block elems   */
  /* QKIND_FFN: y = down( silu(gate(x)) * up(x) ); gate|up is ONE matrix of
   * 2*inter rows (gate rows first), down is [hidden x inter].               */
  int32_t fmt_gateup;      /* QFMT_* for gate|up                             */
  int32_t fmt_down;        /* QFMT_* for down                                */
  int64_t hidden;          /* FFN and MoE hidden size                        */
  int64_t inter;           /* FFN / per-expert intermediate size             */
  /* QKIND_MOE: router fp32 [n_experts x hidden]; experts' gate|up and down
   * are stored as n_experts consecutive matrices of the FFN shapes above,
   * all in fmt_expert; plus one shared expert of the same shape.           */
  int64_t n_experts;       /* routed experts                                 */
  int32_t top_k;           /* experts selected per token (1..16)             */
  int32_t fmt_expert;      /* QFMT_* of every expert matrix                  */
  /* QFMT_IQ4_NL and QFMT_IQ4_XS only: host pointer to 16 int8 codebook
   * entries sorted ascending, copied at plan creation (not kept).          */
  const int8_t *codebook16;
} qgemv_desc;

typedef struct qgemv_plan *qgemv_t;

/* Create a plan: the descriptor (kind, version, format, shapes, codebook)
 * is validated and copied into a host-side handle. A plan is the "load once,
 * then call per token" half of the pure-C device module in "01 · Phase
 * overview: from 2B to 8B to MoE" (icman.com.cn, section 一 and ledger item
 * ①); the format and shape fields describe the packed GGUF-style blocks of
 * "Why expert caching can't save dense models" (xhh.club, Q&A on computing
 * GGUF blocks without FP16 expansion). *out is NULL on failure. Errors:
 * QGEMV_EINVAL (null argument, unknown kind, missing or unsorted codebook),
 * QGEMV_EVERSION, QGEMV_EFORMAT, QGEMV_ESHAPE. */
int qgemv_create(qgemv_t *out, const qgemv_desc *desc);
/* Free a plan's host memory (NULL is accepted). Calls already enqueued with
 * the plan are unaffected: nothing on the device refers to it. */
int qgemv_destroy(qgemv_t h);

/* Bytes of caller-allocated device workspace needed for a call with m
 * tokens (1 <= m <= max_m, else QGEMV_ESHAPE). The workspace holds the
 * quantized activations and every intermediate of the call; it is reused
 * across calls and owned by the caller -- the buffer pool that "01 · Phase
 * overview: from 2B to 8B to MoE" (icman.com.cn, ledger item ⑦) keeps off
 * the per-token path, and the single reused workspace of the fused FFN in
 * "Why expert caching can't save dense models" (xhh.club, single-stream
 * fusion section). One workspace per concurrent call. */
int qgemv_workspace_size(qgemv_t h, int m, size_t *bytes);

/* Byte offsets, inside the workspace for m tokens, of the named
 * intermediates (for checking and debugging; the layout is part of the ABI
 * for a given layout version). Returns QGEMV_EINVAL for a name the plan does
 * not have. Names: "xq" (int8 [m, K]), "dx" (fp32 [m, K/32]), "sx" (int32
 * [m, K/32]); FFN adds "gu" (fp32 [m, 2*inter]), "h" (fp32 [m, inter]), "hq",
 * "hd", "hs"; a GEMV workspace for m >= 9 adds "xqt" (the codes again,
 * int8, 1 KB per 32-element block holding 32 token slots: for element group
 * g = e / 8 and token t, the 8 codes sit at byte
 * ((g * 16 + t % 16) * 2 + t / 16) * 8 of the block), "dxt" (fp32
 * [K/32][32]: the scales again, block-major) and "cxt" (fp32 [K/32][32]: each
 * scale times its block's code sum), all written by the quantizer for the
 * batched matrix-core path (token slots m..31 are left as they were); MoE adds "logits"
 * (fp32 [m, n_experts]), "ids" (int32
 * [m, top_k]), "wts" (fp32 [m, top_k]), "gu" (fp32 [m, top_k + 1, 2*inter]),
 * "h", "hq", "hd", "hs" (per token and slot, shared expert last). */
int qgemv_workspace_offset(qgemv_t h, int m, const char *name, size_t *offset);

/* Minimum device allocation for weight buffer `which` of the plan:
 * GEMV 0 = W; FFN 0 = gate|up, 1 = down; MoE 0 = all experts' gate|up,
 * 1 = all experts' down, 2 = shared gate|up, 3 = shared down, 4 = router. */
int qgemv_weight_bytes(qgemv_t h, int which, size_t *bytes);

/* y[m, n] = W . x for a QKIND_GEMV plan (decode GEMV, 1 <= m <= max_m):
 * the activations are quantized on the device to 32-element int8 blocks
 * with an fp32 scale, and each packed weight block is decoded in registers
 * and combined with them by integer dot products, then scaled ("Why expert
 * caching can't save dense models", xhh.club, in-place compute section and
 * its Q&A on computing GGUF blocks without FP16 expansion).
 * x: fp32 [m, k], 16-byte aligned. y: fp32 [m, n]. ws: workspace of at
 * least qgemv_workspace_size(h, m) bytes, 256-byte aligned. Launches on
 * `stream`: for one token with k <= 2048 (k <= 4096 for Q4_0, Q8_0, Q4_K
 * and Q6_K) one GEMV kernel that quantizes x in its prologue; otherwise the
 * activation quantizer, then the format's GEMV kernel. For Q4_K and Q6_K with m >= 9 the block dots run on int8 matrix
 * cores over 32-token tiles (K split across a workgroup's waves, summed in a
 * fixed order); results follow the same rounding contract either way. */
int qgemv_run(qgemv_t h, const void *w, const float *x, float *y, int m,
              void *ws, size_t ws_bytes, void *stream);

/* qgemv_run for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results as qgemv_run, with the workspace taken from
 * a fixed scratch array that the library holds in device memory, one copy
 * per GPU for the life of the process, instead of a caller-allocated one.
 * The call allocates nothing. Limit: the call's workspace
 * (qgemv_workspace_size(h, m)) must fit in 4 MiB, else QGEMV_EWORKSPACE
 * (every m = 1 call fits: k <= 65536 needs 80 KiB). Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (on two streams
 * or from two threads) race and must be serialized by the caller. Other
 * errors as qgemv_run; a failure to find the scratch is QGEMV_EHIP. */
int qgemv_run_noalloc(qgemv_t h, const void *w, const float *x, float *y, int m, void *stream);

/* The two halves of qgemv_run, for callers that apply several GEMVs to one
 * input (quantize once, then run each projection on the same quantized
 * activations -- the same-input projection sharing of "01 · Phase
 * overview", icman.com.cn, ledger item ② and its stage-five fusion result).
 * qgemv_quantize writes the workspace regions "xq", "dx", "sx" for m tokens
 * of x (fp32 [m, k], 16-byte aligned); qgemv_run_quantized reads them and
 * launches only the GEMV kernel. A workspace filled by one plan may be read
 * by another plan with the same k. */
int qgemv_quantize(qgemv_t h, const float *x, int m, void *ws, size_t ws_bytes,
                   void *stream);
int qgemv_run_quantized(qgemv_t h, const void *w, float *y, int m,
                        const void *ws, size_t ws_bytes, void *stream);

/* 16-bit activation variant of qgemv_run for one token: x is quantized to
 * 32-element blocks of int16 codes with an fp32 scale absmax / 32767 (codes
 * rounded half away from zero from the IEEE quotient), a quantization step
 * about 256 times finer than Q8 -- the fix for int8 activation error
 * compounding over a deep MoE stack in "01 · Phase overview: from 2B to 8B
 * to MoE" (icman.com.cn, issue ledger item ⑫). Block dots are int16 x 4- or
 * 5-bit products (exact int32). Supported for QFMT_Q4_K and QFMT_Q5_K plans
 * with k a multiple of 2048 up to 8192 (QGEMV_EFORMAT / QGEMV_ESHAPE
 * otherwise).
 * qgemv_workspace_size_s16 gives the workspace bytes: regions, each 256-byte
 * aligned, "xq" int16 [k] | "dx" fp32 [k/32] | "sx" int32 [k/32], in that
 * order. Launches the 16-bit quantizer, then the GEMV kernel. */
int qgemv_workspace_size_s16(qgemv_t h, size_t *bytes);
int qgemv_run_s16(qgemv_t h, const void *w, const float *x, float *y, void *ws, size_t ws_bytes,
                  void *stream);

/* Float-activation variant of qgemv_run for 1 <= m <= 32 tokens: y[m, n] =
 * x . W_hat^T with x kept in fp32 (no activation quantization) and each
 * weight dequantized exactly (d * code) -- the accuracy variant for the
 * batched (prefill) path, where int8 activations cost about 3 % perplexity
 * and float activations about 0.2 % in "01 · Phase overview: from 2B to 8B
 * to MoE" (icman.com.cn, issue ledger item ⑮). Products and sums are fp32
 * (one to four tokens where x fits in LDS: fp32 vector dot products per
 * 32-element block; otherwise fp32 matrix cores). Supported for QFMT_Q4_0
 * and QFMT_Q8_0 plans
 * (QGEMV_EFORMAT otherwise); m outside 1..32 is QGEMV_ESHAPE (the plan's
 * max_m does not apply: no workspace is used). x: fp32 [m, k], 16-byte
 * aligned; w 16-byte aligned; y: fp32 [m, n]. One kernel on `stream`. */
int qgemv_run_f32act(qgemv_t h, const void *w, const float *x, float *y, int m, void *stream);

/* Fused FFN sublayer for a QKIND_FFN plan, on one stream with one
 * workspace: quantize x -> gate|up GEMV -> h = silu(gate) * up, re-quantized
 * to Q8 -> down GEMV -> y[m, hidden]. The sublayer is queued on a single
 * stream with a reused workspace ("Why expert caching can't save dense
 * models", xhh.club, single-stream fusion section); gate and up run as one
 * projection of the shared input ("01 · Phase overview", icman.com.cn,
 * ledger item ② on fusing gate/up). */
int qffn_run(qgemv_t h, const void *w_gateup, const void *w_down,
             const float *x, float *y, int m, void *ws, size_t ws_bytes,
             void *stream);

/* MoE FFN layer for a QKIND_MOE plan, entirely on the device: fp32 router
 * GEMV of the unquantized x -> top_k by logit (ties to the lower index) ->
 * softmax over the selected logits -> for each selected expert and the
 * shared expert: gate|up GEMV, SwiGLU, re-quantization, down GEMV -> y[t] =
 * sum_k w_k * out_k (slot order) + shared. Expert ids never leave the
 * device ("Understanding Qwen3.6-35B-A3B in llama.cpp", cnblogs, section 1.1
 * on routing; "01 · Phase overview", icman.com.cn, stage three on device
 * router / top-k / softmax and expert kernels). */
int qmoe_run(qgemv_t h, const float *w_router, const void *w_experts_gateup,
             const void *w_experts_down, const void *w_shared_gateup,
             const void *w_shared_down, const float *x, float *y, int m,
             void *ws, size_t ws_bytes, void *stream);

/* qmoe_run with 16-bit activations: x and every expert's h are quantized to
 * 32-element blocks of int16 codes (scale absmax / 32767), the fix the
 * issue ledger of "01 · Phase overview: from 2B to 8B to MoE" (icman.com.cn,
 * item ⑫) applied to its MoE FFN when int8 activation error compounded over
 * 48 layers. Router, top-k, grouping and combine are those of qmoe_run; the
 * expert GEMVs run on int16 x 4-bit products. Needs QFMT_Q4_0 experts
 * (QGEMV_EFORMAT) with hidden and inter in {512, 1024, 2048, 4096}
 * (QGEMV_ESHAPE). Same workspace as qmoe_run: it also writes the regions
 * "xq16" (int16 [m, hidden]) and "hq16" (int16 [m*(top_k+1), inter]); "dx",
 * "sx", "hd", "hs" then hold the 16-bit blocks' scales and sums. */
int qmoe_run_s16(qgemv_t h, const float *w_router, const void *w_experts_gateup,
                 const void *w_experts_down, const void *w_shared_gateup,
                 const void *w_shared_down, const float *x, float *y, int m,
                 void *ws, size_t ws_bytes, void *stream);

/* Human-readable text of a status code (static string). */
const char *qgemv_status_string(int status);
/* Message of the calling thread's last failed call ("" if none). */
const char *qgemv_last_error(void);

/* ---- checking exports: same device code as the production kernels, with
 * a different epilogue. ---- */

/* The activation quantizer alone: x fp32 [m, k] -> xq int8 [m, k], dx fp32
 * [m, k/32], sx int32 [m, k/32] (block sums). k multiple of 32. */
int qgemv_debug_quantize(const float *x, int8_t *xq, float *dx, int32_t *sx,
                         int m, int64_t k, void *stream);

/* Exact per-block integer dot products of a GEMV plan's weights with
 * quantized activations xq int8 [m, k]: dots int32 [m, n, k/32] with
 * Q4_0: sum xq*(q-8); Q8_0: sum xq*q; IQ4_NL: sum xq*cb[q]; Q4_K: sum xq*q
 * per 32-element sub-block; and for Q6_K dots int32 [m, n, k/16] =
 * sum xq*(q-32) per 16-element sub-block. Runs the production kernel the
 * plan uses for m tokens (staging and decode) with an integer-store
 * epilogue. ws/ws_bytes: a workspace of qgemv_workspace_size(h, m) bytes,
 * used (its "xqt" region) only when m >= 9 and the format is Q4_K or Q6_K;
 * may be NULL/0 otherwise. */
int qgemv_debug_block_dots(qgemv_t h, const void *w, const int8_t *xq,
                           int32_t *dots, int m, void *ws, size_t ws_bytes,
                           void *stream);

/* The 16-bit quantizer alone: x fp32 [m, k] -> xq int16 [m, k], dx fp32
 * [m, k/32], sx int32 [m, k/32]. k multiple of 32. */
int qgemv_debug_quantize_s16(const float *x, int16_t *xq, float *dx, int32_t *sx, int m, int64_t k,
                             void *stream);

/* Exact per-sub-block dots of a Q4_K or Q5_K plan's weights with 16-bit codes xq
 * int16 [k] (one token): dots int32 [n, k/32] = sum xq*q per 32-element
 * sub-block, from the production 16-bit GEMV kernel with an integer-store
 * epilogue. Same shape limits as qgemv_run_s16. */
int qgemv_debug_block_dots_s16(qgemv_t h, const void *w, const int16_t *xq, int32_t *dots, void *stream);

/* Forget the cached launch facts of every kernel on every device (the next
 * launch of each kernel queries them again). For tests that need a kernel's
 * first use to happen at a chosen point (inside stream capture, from several
 * threads at once). Never needed for correctness. */
int qgemv_debug_clear_launch_cache(void);

/* Streaming-read measurement: reads `bytes` bytes of device memory at `buf`
 * once, with the load shape of the GEMV kernels (16-byte non-temporal
 * vector loads, several in flight per lane, workgroups on every compute
 * unit), and computes nothing from them. Timing it at a matrix's size gives
 * the read rate a GEMV of that matrix could reach at best (the pages drill
 * down to such a single-kernel access-pattern test: "01 · Phase overview:
 * from 2B to 8B to MoE", icman.com.cn, issue ledger). buf and bytes need
 * 16-byte alignment; `out` is one device uint32 that is written only if the
 * data xor-reduce to one fixed constant (so that the loads cannot be
 * dropped); its value means nothing. Asynchronous on `stream`. */
int qgemv_debug_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMV_H */
