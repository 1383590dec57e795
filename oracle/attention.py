"""Decode attention for one new token over a KV cache, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the GPU path computes, stated as its plain definition: for every query
head h, with the key/value head it shares g = h // (Hq / Hkv) (grouped-query
attention), scores s_t = (q_h . k_{g,t}) * scale over the T cached tokens,
softmax weights p_t = exp(s_t - max_u s_u) / sum_u exp(s_u - max_u s_u) and
output o_h = sum_t p_t v_{g,t}.

The long-context attention of "Why expert caching can't save dense models:
running a 27B dense model in 16 GB VRAM" (xhh.club, section on in-place
compute and single-stream fusion, and its Q&A on long-context attention)
splits the tokens into chunks, computes each chunk's partial result and
merges the chunks; short contexts use one online-softmax pass. Both are
exact rearrangements of the definition above (up to rounding order), so the
oracle is that definition, computed directly in fp64 with no chunking.

Readings (the pages are silent on these):
  * the cache holds fp16 keys and values, [Hkv, T, D], tokens contiguous per
    head, and the query is fp32 [Hq, D], already position-encoded;
  * scale = 1 / sqrt(D);
  * the output gate of gated attention and the projections around the
    attention core are not part of this kernel.
The head shape used by the workloads (16 query heads, 2 key/value heads,
head dimension 256) is the gated-attention shape in "Understanding
Qwen3.6-35B-A3B in llama.cpp" (cnblogs, section 1.1, model shape list).
"""
from __future__ import annotations

import numpy as np


def decode_attention(q, k, v, scale=None):
    """q [Hq, D] (any float), k and v [Hkv, T, D] (fp16 or wider).
    Returns o [Hq, D] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    hkv, t, d2 = k.shape
    assert d2 == d and v.shape == k.shape and hq % hkv == 0 and t >= 1
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = hq // hkv
    o = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = (k[g] @ q[h]) * scale           # [T]
        e = np.exp(s - s.max())
        p = e / e.sum()
        o[h] = p @ v[g]
    return o
