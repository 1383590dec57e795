/*
 * qattn.h -- C ABI of the decode-attention kernels that run beside the
 * block-quantized GEMVs on the same decode step (AMD MI355X, gfx950).
 *
 * Computes, for one new token, o_h = softmax(q_h . K_g^T / sqrt(D)) V_g for
 * every query head h, where g = h / (n_heads / n_kv_heads) is the key/value
 * head that h shares (grouped-query attention). Long contexts are split into
 * chunks whose partial softmax results (running maximum, sum of exponentials,
 * unnormalised output) are merged in a second pass; short contexts take a
 * single online-softmax pass. This is the two-stage chunked attention of
 * "Why expert caching can't save dense models: running a 27B dense model in
 * 16 GB VRAM" (xhh.club, in-place compute and single-stream fusion section
 * and its Q&A on long-context attention). The workload head shape (16 query
 * heads, 2 key/value heads, dimension 256) is the gated-attention shape in
 * "Understanding Qwen3.6-35B-A3B in llama.cpp" (cnblogs, section 1.1).
 *
 * Conventions are those of qgemv.h: 0 (QGEMV_OK) or a negative QGEMV_E*
 * status, validation on the host before anything is enqueued, device
 * pointers owned by the caller, no allocation, no synchronization,
 * qgemv_last_error() for the message of the last failure on this thread.
 */
#ifndef QATTN_H
#define QATTN_H

#include <stddef.h>
#include <stdint.h>

#include "qgemv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes qattn_decode needs for this shape (0 when the context is
 * short enough for the single pass; the workspace pointer may then be NULL).
 * Shape limits: head_dim 128 or 256; n_heads a multiple of n_kv_heads with
 * n_heads / n_kv_heads in {1, 2, 4, 8}; 1 <= n_ctx and
 * n_ctx * head_dim * 2 + 4096 < 2^31. Returns QGEMV_ESHAPE otherwise. */
int qattn_workspace_size(int n_heads, int n_kv_heads, int head_dim, int64_t n_ctx, size_t *bytes);

/* out[h, :] = attention of query head h over the n_ctx cached tokens.
 *   q        fp32 [n_heads, head_dim], device, 16-byte aligned (already
 *            position-encoded; scaled by 1/sqrt(head_dim) inside).
 *   k_cache  fp16 (IEEE binary16 bits) [n_kv_heads, n_ctx, head_dim],
 *   v_cache  same layout; device, 16-byte aligned, tokens contiguous per head.
 *   out      fp32 [n_heads, head_dim], device, 16-byte aligned.
 *   ws       device workspace of at least qattn_workspace_size() bytes,
 *            256-byte aligned (ignored when that size is 0). Its contents
 *            are overwritten; calls that share a workspace must not overlap.
 * Errors: QGEMV_EINVAL (null pointer), QGEMV_EALIGN, QGEMV_ESHAPE,
 * QGEMV_EWORKSPACE, QGEMV_EHIP (launch refused). */
int qattn_decode(const float *q, const void *k_cache, const void *v_cache, float *out, int n_heads,
                 int n_kv_heads, int head_dim, int64_t n_ctx, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QATTN_H */
