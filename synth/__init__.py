"""Seeded synthetic inputs for the block-quantized GEMV, FFN and MoE workloads
(and the decode-attention workload that runs beside them).

This module is shared by the GPU tests, the benchmark and the CPU oracle's
tests. It only draws random numbers and places them at the byte positions of
the block layouts; it contains none of the method's arithmetic (no decode, no
dot product, no scaling). Every generator takes an explicit seed and uses
numpy's PCG64 (`numpy.random.default_rng`), with a fixed draw order.

Byte layouts written here (all little-endian, fp16 = IEEE binary16):

  Q4_0    32 elements, 18 B: d fp16 | 16 B of packed 4-bit codes
  Q8_0    32 elements, 34 B: d fp16 | 32 int8 codes in -127..127
  IQ4_NL  32 elements, 18 B: d fp16 | 16 B of packed 4-bit codebook indices
  Q4_K   256 elements, 144 B: d fp16 | dmin fp16 | 12 B of sixteen 6-bit fields
                               | 128 B of packed 4-bit codes
  Q6_K   256 elements, 210 B: d fp16 | 16 int8 sub-block scales in -64..63
                               | 128 B low code bits | 64 B high code bits
  Q5_K   256 elements, 176 B: d fp16 | dmin fp16 | 12 B of sixteen 6-bit fields
                               | 32 B fifth code bits | 128 B packed 4-bit codes
  IQ4_XS 256 elements, 136 B: d fp16 | 2 B + 4 B of eight 6-bit sub-scales
                               | 128 B of packed 4-bit codebook indices

Because every code field is a whole number of uniformly random bits, drawing
uniform random bytes for the packed regions gives codes that are uniform over
their full range, whatever the bit order inside the bytes. Only fields with a
restricted range (the fp16 scales, Q8_0's int8 codes, Q6_K's int8 scales) are
drawn field by field.

Distributions follow the workload descriptions of the decode GEMV study that
this library implements: scales d (and Q4_K's dmin) uniform in [1e-3, 1e-2]
stored as fp16 (round to nearest even), activations N(0, 1) in fp32, Q4_K
scale and min fields uniform in 0..63, Q8_0 codes uniform in -127..127, Q6_K
scales uniform in -64..63 and codes uniform in 0..63. Q5_K follows Q4_K
(codes uniform in 0..31); IQ4_XS sub-scales are uniform 6-bit fields.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "FORMATS", "BLOCK_ELEMS", "BLOCK_BYTES", "row_bytes", "padded_bytes",
    "activations", "weights", "codebook", "router_weights", "moe_experts", "attention_inputs",
]

FORMATS = ("q4_0", "q8_0", "q4_k", "q6_k", "iq4_nl", "q5_k", "iq4_xs")
BLOCK_ELEMS = {"q4_0": 32, "q8_0": 32, "iq4_nl": 32, "q4_k": 256, "q6_k": 256, "q5_k": 256,
               "iq4_xs": 256}
BLOCK_BYTES = {"q4_0": 18, "q8_0": 34, "iq4_nl": 18, "q4_k": 144, "q6_k": 210, "q5_k": 176,
               "iq4_xs": 136}

# Byte offset of fields with a restricted range inside one block.
_D_OFF = 0          # fp16 d, every format
_DMIN_OFF_Q4K = 2   # fp16 dmin, Q4_K and Q5_K
_Q8_CODES = (2, 34)
_Q6K_SC = (2, 18)


def row_bytes(fmt: str, k: int) -> int:
    be = BLOCK_ELEMS[fmt]
    if k <= 0 or k % be:
        raise ValueError(f"{fmt}: K={k} is not a positive multiple of {be}")
    return (k // be) * BLOCK_BYTES[fmt]


def padded_bytes(fmt: str, n: int, k: int) -> int:
    """Bytes of an N-row matrix, rounded up to 16 (128-bit loads may read the tail)."""
    b = n * row_bytes(fmt, k)
    return (b + 15) // 16 * 16


def _fp16_uniform(rng, shape, lo=1e-3, hi=1e-2):
    return rng.uniform(lo, hi, size=shape).astype(np.float32).astype(np.float16)


def activations(seed: int, m: int, k: int) -> np.ndarray:
    """fp32 activations x[m, k] ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((m, k), dtype=np.float64).astype(np.float32)


def weights(fmt: str, n: int, k: int, seed: int, *, fixed_d: float | None = None,
            fixed_dmin: float | None = None, fill: int | None = None) -> np.ndarray:
    """Packed weight matrix as uint8[padded_bytes] (rows of blocks, row-major).

    fixed_d / fixed_dmin replace the random scales by one constant (stored as
    fp16); fill replaces every random packed byte by one constant byte. These
    exist to build structured cases (unit scales, constant codes) from the
    same byte layout.
    """
    rng = np.random.default_rng(seed)
    be, bb = BLOCK_ELEMS[fmt], BLOCK_BYTES[fmt]
    nb = row_bytes(fmt, k) // bb
    blk = rng.integers(0, 256, size=(n, nb, bb), dtype=np.uint8)
    if fill is not None:
        blk[...] = np.uint8(fill)
    if fmt == "q8_0":
        lo, hi = _Q8_CODES
        codes = rng.integers(-127, 128, size=(n, nb, hi - lo), dtype=np.int16).astype(np.int8)
        if fill is None:
            blk[..., lo:hi] = codes.view(np.uint8)
    if fmt == "q6_k":
        lo, hi = _Q6K_SC
        sc = rng.integers(-64, 64, size=(n, nb, hi - lo), dtype=np.int16).astype(np.int8)
        if fill is None:
            blk[..., lo:hi] = sc.view(np.uint8)
    d = _fp16_uniform(rng, (n, nb)) if fixed_d is None else np.full((n, nb), fixed_d, np.float16)
    blk[..., _D_OFF:_D_OFF + 2] = d.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    if fmt in ("q4_k", "q5_k"):
        dm = _fp16_uniform(rng, (n, nb)) if fixed_dmin is None else np.full((n, nb), fixed_dmin, np.float16)
        blk[..., _DMIN_OFF_Q4K:_DMIN_OFF_Q4K + 2] = dm.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    out = np.zeros(padded_bytes(fmt, n, k), np.uint8)
    out[: blk.size] = blk.reshape(-1)
    return out


def codebook(seed: int) -> np.ndarray:
    """Sorted int8[16] IQ4_NL codebook: -127 and 113 at the ends, 14 distinct
    interior values drawn without replacement from -126..112."""
    rng = np.random.default_rng(seed)
    inner = rng.choice(np.arange(-126, 113), size=14, replace=False)
    cb = np.sort(np.concatenate([[-127, 113], inner])).astype(np.int8)
    return cb


def router_weights(seed: int, n_experts: int, hidden: int) -> np.ndarray:
    """fp32 router matrix [n_experts, hidden] ~ N(0, 1/hidden), so that
    router logits for N(0, 1) activations are roughly N(0, 1)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n_experts, hidden)) / np.sqrt(hidden)
    return w.astype(np.float32)


def moe_experts(seed: int, n_experts: int, hidden: int, inter: int, fmt: str = "q4_0"):
    """Packed expert weights.

    Returns (gateup, down): gateup is n_experts contiguous [2*inter x hidden]
    matrices (gate rows first, then up rows); down is n_experts contiguous
    [hidden x inter] matrices. Each is a flat uint8 array padded to 16 bytes.
    """
    rng = np.random.default_rng(seed)
    s1, s2 = rng.integers(0, 2**31, size=2)
    gu_one = n_experts * 2 * inter
    gu = weights(fmt, gu_one, hidden, int(s1))
    dn = weights(fmt, n_experts * hidden, inter, int(s2))
    return gu, dn


def attention_inputs(seed: int, n_heads: int, n_kv_heads: int, head_dim: int, n_ctx: int):
    """Decode-attention inputs: q fp32 [n_heads, head_dim] ~ N(0, 1); keys and
    values fp16 [n_kv_heads, n_ctx, head_dim] ~ N(0, 1) rounded to fp16
    (draw order: q, k, v)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_heads, head_dim)).astype(np.float32)
    k = rng.standard_normal((n_kv_heads, n_ctx, head_dim)).astype(np.float16)
    v = rng.standard_normal((n_kv_heads, n_ctx, head_dim)).astype(np.float16)
    return q, k, v
