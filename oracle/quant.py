"""Q8 activation quantizer (and its 16-bit variant), written out from its
definition.

The method quantizes activations on the device into 32-element int8 blocks
with one fp32 scale per block ("Why expert caching can't save dense models",
xhh.club: the Q&A on computing GGUF blocks in place, and the in-place compute
section, which names the Q8 activation format with an fp32 scale). The scale
is the block's absolute maximum over 127 and codes round half away from zero
(the decode-GEMV workload description).

Readings where the pages are silent:
* The scale is d = fl32(a / 127) (IEEE binary32 division, round to nearest
  even) and codes are taken from v = fl32(x / d), i.e. a true division, not a
  multiplication by a reciprocal.
* Round half away from zero is applied to the fp32 value v, evaluated exactly
  in fp64 as sign(v) * floor(|v| + 0.5); codes are clamped to [-127, 127].
* A block whose absolute maximum is 0 gets d = 0 and all codes 0.
* The block sum s = sum(q) is returned too; it is an exact integer function of
  the codes and is used by formats with an offset or a min term.
"""
from __future__ import annotations

import numpy as np

QK = 32


def _quantize_blocks(x, qmax, dtype):
    """32-element blocks: d = fl32(absmax / qmax), q = round-half-away(fl32(x / d))
    clamped to [-qmax, qmax], s = sum(q); an all-zero block gives d = 0, q = 0."""
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("activations must be float32")
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    if k % QK:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(m, k // QK, QK)
    a = np.max(np.abs(xb), axis=-1)                      # exact in fp32
    nz = a > 0
    d = np.where(nz, a / np.float32(qmax), np.float32(0)).astype(np.float32)
    dsafe = np.where(nz, d, np.float32(1)).astype(np.float32)
    v = (xb / dsafe[..., None]).astype(np.float32)       # fp32 division, RNE
    v64 = v.astype(np.float64)
    q = np.sign(v64) * np.floor(np.abs(v64) + 0.5)        # half away from zero
    q = np.clip(q, -qmax, qmax)
    q = np.where(nz[..., None], q, 0).astype(dtype)
    s = q.astype(np.int32).sum(axis=-1, dtype=np.int32)
    return q.reshape(m, k), d, s


def quantize_q8(x):
    """Quantize fp32 activations x[m, k] (k a multiple of 32) to Q8 blocks.

    Returns (xq int8[m, k], dx float32[m, k/32], sx int32[m, k/32]).
    """
    return _quantize_blocks(x, 127, np.int8)


def quantize_s16(x):
    """16-bit variant: the same 32-element blocks with an fp32 scale, codes
    int16 with d = fl32(absmax / 32767), so the quantization step is about
    256 times finer than Q8's ("01 · Phase overview: from 2B to 8B to MoE",
    icman.com.cn, issue ledger item ⑫: int8 activation error compounding over
    a deep MoE stack, fixed by 16-bit activations with a 256x smaller step).
    The rounding, clamping and zero-block readings are those of Q8 above.

    Returns (xq int16[m, k], dx float32[m, k/32], sx int32[m, k/32]).
    """
    return _quantize_blocks(x, 32767, np.int16)


def dequantize_q8(xq, dx):
    """x_hat = dx * xq in fp64 (exact: fp32 times a small integer; also used
    for the 16-bit codes)."""
    xq = np.asarray(xq)
    m, k = xq.shape
    return (xq.reshape(m, k // QK, QK).astype(np.float64)
            * np.asarray(dx, np.float64)[..., None]).reshape(m, k)
