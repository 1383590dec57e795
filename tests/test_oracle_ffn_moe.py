"""Pins for the oracle's SwiGLU / FFN chain and its MoE router and combine."""
import math

import numpy as np
import pytest

import synth
from oracle import ffn, formats, moe
from oracle.quant import quantize_q8, dequantize_q8


def test_silu_closed_forms():
    assert ffn.silu(0.0) == 0.0
    assert ffn.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(ffn.silu(-40.0)) < 1e-15
    z = np.linspace(-12, 12, 97)
    # z*s(z) - (-z)*s(-z) = z (s(z) + s(-z)) = z
    assert np.allclose(ffn.silu(z) - ffn.silu(-z), z, rtol=0, atol=1e-14)
    for v in (-3.5, -0.25, 0.7, 2.0):
        assert ffn.silu(v) == pytest.approx(v / (1 + math.exp(-v)), rel=1e-15)


def test_swiglu_gate_first():
    gu = np.array([[1.0, -2.0, 3.0, 4.0]])
    h = ffn.swiglu(gu, 2)
    assert np.allclose(h, [[ffn.silu(1.0) * 3.0, ffn.silu(-2.0) * 4.0]])


def test_ffn_identity_down_returns_requantized_h():
    # Q6_K down with d = 1, sc = 1, q = 33 on the diagonal and 32 elsewhere is
    # W_down = [I | 0]; then y equals the dequantized requantized h[:H].
    H, I = 256, 512
    gu_raw = synth.weights("q4_k", 2 * I, H, seed=3)
    nb = I // 256
    q = np.full((H, nb, 256), 32, np.int64).reshape(H, I)
    q[np.arange(H), np.arange(H)] = 33
    down = formats.encode("q6_k", {"d": np.ones((H, nb)), "sc": np.ones((H, nb, 16), np.int64),
                                   "q": q.reshape(H, nb, 256)})
    x = synth.activations(4, 1, H)
    r = ffn.ffn_ref(gu_raw, down, x, H, I)
    hh = dequantize_q8(r["hq"], r["hd"])
    assert np.array_equal(r["y"], hh[:, :H])


def test_router_topk_brute_force_and_ties():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal((5, 256))
    lg[2, 10] = lg[2, 20] = lg[2, 30] = 9.0          # three-way tie at the top
    ids = moe.topk(lg, 8)
    for t in range(5):
        full = sorted(range(256), key=lambda j: (-lg[t, j], j))
        assert list(ids[t]) == full[:8]
    assert list(ids[2, :3]) == [10, 20, 30]
    w = moe.topk_weights(lg, ids)
    assert np.allclose(w.sum(1), 1.0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)
    # softmax over the selected = full softmax renormalised over the selected
    full = np.exp(lg - lg.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ids, 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    # shift invariance
    assert np.allclose(moe.topk_weights(lg + 3.25, ids), w, rtol=1e-13)
    assert np.array_equal(moe.topk(lg + 3.25, 8), ids)


def test_router_logits_match_plain_matmul():
    wr = synth.router_weights(1, 256, 2048)
    x = synth.activations(2, 3, 2048)
    lg = moe.router_logits(wr, x)
    assert np.allclose(lg, x.astype(np.float64) @ wr.astype(np.float64).T, rtol=0, atol=1e-12)
    assert 0.5 < lg.std() < 2.0          # N(0, 1/H) weights give ~N(0, 1) logits


def test_moe_identical_experts_reduce_to_one_expert_plus_shared():
    H, I, E, K = 256, 64, 16, 4
    one_gu = synth.weights("q4_0", 2 * I, H, seed=5)
    one_dn = synth.weights("q4_0", H, I, seed=6)
    gu_all = np.tile(one_gu, E)
    dn_all = np.tile(one_dn, E)
    sh_gu = synth.weights("q4_0", 2 * I, H, seed=7)
    sh_dn = synth.weights("q4_0", H, I, seed=8)
    wr = synth.router_weights(2, E, H)
    x = synth.activations(3, 2, H)
    r = moe.moe_ref(wr, gu_all, dn_all, sh_gu, sh_dn, x, H, I, K)
    for t in range(2):
        xq, dx, _ = quantize_q8(x[t:t + 1])
        e = moe.expert_chain(one_gu, one_dn, xq, dx, H, I)["out"][0]
        s = moe.expert_chain(sh_gu, sh_dn, xq, dx, H, I)["out"][0]
        assert np.allclose(r["y"][t], e + s, rtol=1e-13, atol=1e-15)
