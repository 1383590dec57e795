"""The quantized GEMV y = W_hat . x_hat, in two independent forms.

The method reads packed weight blocks in place, never building a
dequantized copy of the matrix, and accumulates int8 dot products between
the quantized activations and the decoded block codes, then applies the
block scales and, for the K-quant super-blocks, the min correction ("Why
expert caching can't save dense models", xhh.club, Q&A on computing GGUF
blocks in place; the CPU reference of "01 · Phase overview: from 2B to 8B to
MoE", icman.com.cn, dequantizes row by row and takes dot products).

Mathematically the result is exactly y = W_hat . x_hat, with W_hat the
decoded weights and x_hat = dx * xq the dequantized activations, up to the
order of floating-point rounding. So:

* `gemv_dequant` (graded reference) is that plain definition: decode to fp64,
  form x_hat in fp64, one fp64 matmul (row chunks bound the memory).
* `block_dots` gives the exact integer quantity of each (row, block) pair.
* `gemv_intdot` rebuilds y from those integers and the scales in fp64; it must
  agree with `gemv_dequant` to fp64 rounding.

Per-block integer quantities (int64 here; all fit in int32):
  q4_0    D = sum xq * (q - 8)        per 32-element block      [m, n, k/32]
  q8_0    D = sum xq * q              per 32-element block      [m, n, k/32]
  iq4_nl  D = sum xq * cb[q]          per 32-element block      [m, n, k/32]
  q4_k    D = sum xq * q              per 32-element sub-block  [m, n, k/32]
          (the min term uses the activation block sum sx)
  q6_k    P = sum xq * (q - 32)       per 16-element sub-block  [m, n, k/16]
  q5_k    D = sum xq * q              per 32-element sub-block  [m, n, k/32]
          (q in 0..31; the min term as for q4_k)
  iq4_xs  D = sum xq * cb[q]          per 32-element sub-block  [m, n, k/32]
          (the sub-block scale is d * (ls - 32))
"""
from __future__ import annotations

import numpy as np

from . import formats
from .quant import quantize_q8, dequantize_q8

ROW_CHUNK = 4096


def _codes(fmt, f, codebook):
    """Signed integer code per element that multiplies xq in the block dot."""
    if fmt == "q4_0":
        return f["q"] - 8
    if fmt == "q8_0":
        return f["q"]
    if fmt in ("iq4_nl", "iq4_xs"):
        return np.asarray(codebook, np.int64)[f["q"]]
    if fmt in ("q4_k", "q5_k"):
        return f["q"]
    if fmt == "q6_k":
        return f["q"] - 32
    raise ValueError(fmt)


def block_dots(fmt, raw, n, k, xq, codebook=None):
    """Exact per-block integer dot products, int64[m, n, k/G] (G = 32, or 16 for q6_k)."""
    xq = np.asarray(xq, np.int64)
    if xq.ndim == 1:
        xq = xq[None]
    m = xq.shape[0]
    g = 16 if fmt == "q6_k" else 32
    out = np.empty((m, n, k // g), np.int64)
    rb = formats.row_bytes(fmt, k)
    raw = np.asarray(raw, np.uint8).reshape(-1)
    xg = xq.reshape(m, k // g, g)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        f = formats.decode(fmt, raw[r0 * rb:r1 * rb], r1 - r0, k)
        c = _codes(fmt, f, codebook).reshape(r1 - r0, k // g, g)
        out[:, r0:r1, :] = np.einsum("tbi,rbi->trb", xg, c)
    return out


def gemv_dequant(fmt, raw, n, k, xq, dx, codebook=None):
    """y[m, n] = x_hat . W_hat^T in fp64, from decoded fp64 weights."""
    xh = dequantize_q8(np.atleast_2d(xq), np.atleast_2d(dx))        # [m, k] fp64
    m = xh.shape[0]
    y = np.empty((m, n), np.float64)
    rb = formats.row_bytes(fmt, k)
    raw = np.asarray(raw, np.uint8).reshape(-1)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        w = formats.values(fmt, raw[r0 * rb:r1 * rb], r1 - r0, k, codebook)
        y[:, r0:r1] = xh @ w.T
    return y


def gemv_intdot(fmt, raw, n, k, xq, dx, sx, codebook=None):
    """y[m, n] from the exact integer block dots and fp64 scales."""
    xq = np.atleast_2d(xq)
    dx = np.atleast_2d(np.asarray(dx, np.float64))
    sx = np.atleast_2d(np.asarray(sx, np.int64))
    m = xq.shape[0]
    y = np.empty((m, n), np.float64)
    rb = formats.row_bytes(fmt, k)
    raw = np.asarray(raw, np.uint8).reshape(-1)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        nr = r1 - r0
        part = raw[r0 * rb:r1 * rb]
        f = formats.decode(fmt, part, nr, k)
        D = block_dots(fmt, part, nr, k, xq, codebook).astype(np.float64)
        if fmt in ("q4_0", "q8_0", "iq4_nl"):
            # y = sum_b dx_b * d_b * D_b
            y[:, r0:r1] = np.einsum("tb,rb,trb->tr", dx, f["d"], D)
        elif fmt == "iq4_xs":
            # y = sum_j dx_j * d * (ls_j - 32) * D_j
            nb = k // 256
            d = np.repeat(f["d"], 8, axis=1)
            ls = f["ls"].reshape(nr, nb * 8).astype(np.float64)
            y[:, r0:r1] = np.einsum("tj,rj,trj->tr", dx, d * (ls - 32), D)
        elif fmt in ("q4_k", "q5_k"):
            nb = k // 256
            d = np.repeat(f["d"], 8, axis=1)                    # per sub-block
            dmin = np.repeat(f["dmin"], 8, axis=1)
            sc = f["sc"].reshape(nr, nb * 8).astype(np.float64)
            mm = f["m"].reshape(nr, nb * 8).astype(np.float64)
            t1 = np.einsum("tj,rj,trj->tr", dx, d * sc, D)
            t2 = np.einsum("tj,rj,tj->tr", dx, dmin * mm, sx.astype(np.float64))
            y[:, r0:r1] = t1 - t2
        elif fmt == "q6_k":
            nb = k // 256
            d = np.repeat(f["d"], 16, axis=1)                   # per 16-sub-block
            sc = f["sc"].reshape(nr, nb * 16).astype(np.float64)
            dx16 = np.repeat(dx, 2, axis=1)                     # each 32-block covers 2
            y[:, r0:r1] = np.einsum("tj,rj,trj->tr", dx16, d * sc, D)
        else:
            raise ValueError(fmt)
    return y


def gemv_ref(fmt, raw, n, k, x, codebook=None):
    """Quantize fp32 x[m, k] to Q8, then the dequantize form. Returns (y, xq, dx, sx)."""
    xq, dx, sx = quantize_q8(np.atleast_2d(np.asarray(x, np.float32)))
    return gemv_dequant(fmt, raw, n, k, xq, dx, codebook), xq, dx, sx


def gemv_rows(fmt, raw, n, k, rows, xq, dx, codebook=None):
    """y[:, rows] only (for sampled checks on very large matrices)."""
    rb = formats.row_bytes(fmt, k)
    raw = np.asarray(raw, np.uint8).reshape(-1)
    rows = np.asarray(rows, np.int64)
    sel = raw[: n * rb].reshape(n, rb)[rows].reshape(-1)
    return gemv_dequant(fmt, sel, rows.size, k, xq, dx, codebook)


def fp32_gemv(w, x):
    """Plain fp64 product of an fp32 matrix w[n, k] with fp32 x[m, k] -> [m, n]."""
    return np.atleast_2d(np.asarray(x, np.float64)) @ np.asarray(w, np.float64).T


def gemv_float_act(fmt, raw, n, k, x, codebook=None):
    """Float-activation form: y[m, n] = x . W_hat^T in fp64, with x the fp32
    activations as given (no activation quantization) and W_hat the exact
    dequantized weights. The batched (prefill) path computes this when int8
    activations cost too much accuracy: in "01 · Phase overview: from 2B to
    8B to MoE" (icman.com.cn, issue ledger item ⑮) int8 activations in
    prefill raised perplexity by about 3 %, float activations by about 0.2 %.
    """
    xa = np.atleast_2d(np.asarray(x, np.float32)).astype(np.float64)
    return xa @ formats.values(fmt, raw, n, k, codebook).T

