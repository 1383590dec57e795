"""Pins of the decode-attention oracle (CPU only).

Each pin is fixed by the mathematics of softmax attention, not by re-typing
the oracle: a hand-worked two-token example, the one-token and equal-key
special cases, the grouped-query head mapping, invariances (token order, a
common key offset), the one-hot limit at huge scores, the exactness of the
chunk-and-merge rearrangement the GPU path uses, and a pure-Python brute
force on a tiny case.
"""
import math

import numpy as np

import synth
from oracle.attention import decode_attention


def test_worked_two_token_example():
    # D = 4, scale = 1/2: s0 = 0, s1 = (2 ln 3) * 1 / 2 = ln 3, so the weights
    # are 1/4 and 3/4 and o = v0 / 4 + 3 v1 / 4.
    q = np.array([[2 * math.log(3.0), 0, 0, 0]], dtype=np.float64)
    k = np.zeros((1, 2, 4), dtype=np.float16)
    k[0, 1, 0] = 1
    v = np.array([[[4, 0, 8, -4], [0, 4, 4, 8]]], dtype=np.float16)
    o = decode_attention(q, k, v)
    assert np.allclose(o, [[1, 3, 5, 5]], rtol=0, atol=1e-12)


def test_single_token_returns_its_value():
    q, k, v = synth.attention_inputs(1, 4, 2, 64, 1)
    o = decode_attention(q, k, v)
    for h in range(4):
        assert np.array_equal(o[h], v[h // 2, 0].astype(np.float64))


def test_equal_keys_average_values():
    q, k, v = synth.attention_inputs(2, 2, 1, 32, 9)
    k[:] = k[:, :1]
    o = decode_attention(q, k, v)
    assert np.allclose(o, v.astype(np.float64).mean(axis=1).repeat(2, axis=0), rtol=0, atol=1e-12)


def test_grouped_heads_use_their_kv_head():
    # Hq = 4 over Hkv = 2: heads 0, 1 read kv head 0 and heads 2, 3 kv head 1.
    q, k, v = synth.attention_inputs(3, 4, 2, 16, 7)
    v[0] = 1.0
    v[1] = -2.0
    o = decode_attention(q, k, v)
    assert np.allclose(o[:2], 1.0, atol=1e-12) and np.allclose(o[2:], -2.0, atol=1e-12)


def test_token_order_does_not_matter():
    q, k, v = synth.attention_inputs(4, 4, 2, 32, 50)
    perm = np.random.default_rng(0).permutation(50)
    o1 = decode_attention(q, k, v)
    o2 = decode_attention(q, k[:, perm], v[:, perm])
    assert np.allclose(o1, o2, rtol=0, atol=1e-13)


def test_common_key_offset_cancels():
    # k_t -> k_t + c shifts every score of a head by the same amount.
    q, k, v = synth.attention_inputs(5, 2, 1, 16, 20)
    c = np.random.default_rng(1).standard_normal(16)
    o1 = decode_attention(q, k, v)
    o2 = decode_attention(q, k.astype(np.float64) + c, v)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)


def test_huge_scores_select_the_best_key():
    q, k, v = synth.attention_inputs(6, 1, 1, 64, 30)
    s = k[0].astype(np.float64) @ q[0].astype(np.float64)
    best = int(np.argmax(s))
    gap = np.sort(s)[-1] - np.sort(s)[-2]
    q_big = q * (2000.0 / gap)  # best score exceeds the runner-up by >= 250 after scaling by 1/8
    o = decode_attention(q_big, k, v)
    assert np.all(np.isfinite(o))
    assert np.allclose(o[0], v[0, best].astype(np.float64), rtol=0, atol=1e-12)


def test_chunk_merge_is_exact():
    # Split the tokens into chunks; each chunk keeps its max m_c, its sum l_c
    # of exp(s - m_c) and its unnormalised output; merging with weights
    # exp(m_c - max_c m_c) reproduces the whole-context result.
    q, k, v = synth.attention_inputs(7, 2, 1, 32, 103)
    d = q.shape[1]
    ref = decode_attention(q, k, v)
    for chunk in (1, 8, 50, 103):
        for h in range(2):
            s = k[0].astype(np.float64) @ q[h].astype(np.float64) / math.sqrt(d)
            ms, ls, os_ = [], [], []
            for c0 in range(0, 103, chunk):
                sc = s[c0:c0 + chunk]
                m = sc.max()
                e = np.exp(sc - m)
                ms.append(m)
                ls.append(e.sum())
                os_.append(e @ v[0, c0:c0 + chunk].astype(np.float64))
            mm = max(ms)
            w = [math.exp(m - mm) for m in ms]
            o = sum(wi * oi for wi, oi in zip(w, os_)) / sum(wi * li for wi, li in zip(w, ls))
            assert np.allclose(o, ref[h], rtol=0, atol=1e-13)


def test_brute_force_tiny():
    q, k, v = synth.attention_inputs(8, 2, 1, 3, 4)
    o = decode_attention(q, k, v)
    for h in range(2):
        s = [sum(float(q[h, i]) * float(k[0, t, i]) for i in range(3)) / math.sqrt(3) for t in range(4)]
        e = [math.exp(x) for x in s]
        z = sum(e)
        for i in range(3):
            want = sum(e[t] / z * float(v[0, t, i]) for t in range(4))
            assert abs(o[h, i] - want) <= 1e-13
