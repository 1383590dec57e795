"""MoE FFN layer: fp32 router, softmax, top-k, expert chains, combine.

A router scores every expert for the token and only the selected experts run
("Understanding Qwen3.6-35B-A3B in llama.cpp", cnblogs, section 1.1: a router
picks a few experts per token; the model has hidden size 2048, 256 experts
with 8 routed plus 1 shared active, expert intermediate size 512). The device
path runs router, top-k, softmax and the expert gate/up, SwiGLU and down
projections on the GPU and aggregates the weighted outputs ("01 · Phase
overview: from 2B to 8B to MoE", icman.com.cn, stage three and ledger items
on the MoE decode branch).

Readings:
* Router logits are an fp32 GEMV of the unquantized fp32 activations; here
  they are computed in fp64.
* The top-k experts are those with the largest logits; ties go to the lower
  expert index; slots are ordered by descending logit.
* Weights are the softmax over the selected k logits, which equals the
  softmax over all experts renormalised over the k selected.
* The shared expert has the shape and format of a routed expert and is added
  with weight 1.
* Every expert of a token uses that token's single Q8 quantization of x; each
  expert's h is re-quantized to Q8 before its down projection. The 16-bit
  variant (quant=quantize_s16) uses the 16-bit rule for both ("01 · Phase
  overview: from 2B to 8B to MoE", icman.com.cn, issue ledger item ⑫).
* The combine sums slots 0..k-1 in order, then adds the shared expert.
"""
from __future__ import annotations

import numpy as np

from .ffn import swiglu
from .gemv import gemv_dequant
from .quant import quantize_q8


def router_logits(w_router, x):
    """logits[m, E] = x . W_r^T in fp64 (x unquantized fp32)."""
    return (np.atleast_2d(np.asarray(x, np.float64))
            @ np.asarray(w_router, np.float64).T)


def topk(logits, k):
    """ids[m, k] by descending logit, ties to the lower index."""
    logits = np.atleast_2d(logits)
    m, e = logits.shape
    ids = np.empty((m, k), np.int64)
    for t in range(m):
        order = sorted(range(e), key=lambda j: (-logits[t, j], j))
        ids[t] = order[:k]
    return ids


def topk_weights(logits, ids):
    """Softmax over the selected logits, in fp64."""
    sel = np.take_along_axis(np.atleast_2d(logits), ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def expert_chain(w_gu, w_dn, xq, dx, hidden, inter, fmt="q4_0", quant=quantize_q8):
    """One expert on quantized input: returns dict(gu, h, hq, hd, hs, out).
    quant re-quantizes h (Q8, or the 16-bit variant)."""
    gu = gemv_dequant(fmt, w_gu, 2 * inter, hidden, xq, dx)
    h = swiglu(gu, inter)
    hq, hd, hs = quant(h.astype(np.float32))
    out = gemv_dequant(fmt, w_dn, hidden, inter, hq, hd)
    return {"gu": gu, "h": h, "hq": hq, "hd": hd, "hs": hs, "out": out}


def expert_down(w_dn, hq, hd, hidden, inter, fmt="q4_0"):
    return gemv_dequant(fmt, w_dn, hidden, inter, hq, hd)


def combine(outs, w, shared_out):
    """y = sum_k w_k * out_k (slot order) + shared_out."""
    y = np.zeros_like(np.asarray(shared_out, np.float64))
    for kk in range(len(outs)):
        y = y + w[kk] * np.asarray(outs[kk], np.float64)
    return y + shared_out


def moe_ref(w_router, gu_all, dn_all, gu_shared, dn_shared, x, hidden, inter, top_k,
            fmt="q4_0", quant=quantize_q8):
    """Fully independent chain for every token. Returns dict of stages."""
    from .formats import row_bytes as _rb
    x = np.atleast_2d(np.asarray(x, np.float32))
    m = x.shape[0]
    rb_gu, rb_dn = _rb(fmt, hidden), _rb(fmt, inter)
    sz_gu, sz_dn = 2 * inter * rb_gu, hidden * rb_dn
    logits = router_logits(w_router, x)
    ids = topk(logits, top_k)
    w = topk_weights(logits, ids)
    y = np.zeros((m, hidden), np.float64)
    for t in range(m):
        xq, dx, _ = quant(x[t:t + 1])
        outs = []
        for kk in range(top_k):
            e = int(ids[t, kk])
            ch = expert_chain(gu_all[e * sz_gu:(e + 1) * sz_gu], dn_all[e * sz_dn:(e + 1) * sz_dn],
                              xq, dx, hidden, inter, fmt, quant)
            outs.append(ch["out"][0])
        sh = expert_chain(gu_shared, dn_shared, xq, dx, hidden, inter, fmt, quant)["out"][0]
        y[t] = combine(outs, w[t], sh)
    return {"logits": logits, "ids": ids, "w": w, "y": y}
