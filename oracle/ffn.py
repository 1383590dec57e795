"""Fused FFN sublayer: gate|up projection, SwiGLU, re-quantization, down.

The method queues the whole FFN sublayer on one stream and reuses one
workspace ("Why expert caching can't save dense models", xhh.club, in-place
compute and single-stream fusion section); gate and up share the same input
and run as one projection ("01 · Phase overview: from 2B to 8B to MoE",
icman.com.cn, ledger item on fusing QKV and gate/up). The dense workload is
hidden 4096, intermediate 12288, Q4_K gate and up, Q6_K down, with SwiGLU
silu(gate) * up re-quantized to Q8 before the down projection.

Readings:
* gate|up is one matrix of 2*I rows: rows [0, I) are gate, [I, 2I) are up.
* silu(z) = z / (1 + exp(-z)), evaluated in fp64 here.
* The re-quantization of h uses the same Q8 rule as the input activations,
  applied to h rounded to fp32 (the device holds h in fp32).

Each stage is exposed on its own so that a device result can be checked
stage by stage, conditioned on the device's own intermediates where a
floating-point near-tie decides an integer code.
"""
from __future__ import annotations

import numpy as np

from .gemv import gemv_dequant
from .quant import quantize_q8


def silu(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(gu, inter):
    """h = silu(gate) * up in fp64 from gu[m, 2I] (gate first)."""
    gu = np.atleast_2d(np.asarray(gu, np.float64))
    return silu(gu[:, :inter]) * gu[:, inter:2 * inter]


def ffn_ref(w_gateup, w_down, x, hidden, inter, fmt_gateup="q4_k", fmt_down="q6_k"):
    """Fully independent fp64 chain. Returns a dict of every stage."""
    x = np.atleast_2d(np.asarray(x, np.float32))
    xq, dx, sx = quantize_q8(x)
    gu = gemv_dequant(fmt_gateup, w_gateup, 2 * inter, hidden, xq, dx)
    h = swiglu(gu, inter)
    h32 = h.astype(np.float32)
    hq, hd, hs = quantize_q8(h32)
    y = gemv_dequant(fmt_down, w_down, hidden, inter, hq, hd)
    return {"xq": xq, "dx": dx, "sx": sx, "gu": gu, "h": h, "h32": h32,
            "hq": hq, "hd": hd, "hs": hs, "y": y}
