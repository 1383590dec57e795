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


# ---------------------------------------------------------------- router --
# The router is an fp32 GEMV of the unquantized activations. These pins fix
# its arithmetic without recomputing the same product: one-hot activations
# must return the columns of W_r (a transposed operand or a wrong axis fails
# on the square case), basis-vector rows must return single scaled
# activation entries, and small integer operands must match a brute-force sum
# of exact Python integers.

def test_router_logits_one_hot_returns_columns():
    for E, H in ((16, 16), (5, 64)):
        wr = synth.router_weights(11, E, H)
        x = np.eye(H, dtype=np.float32)[: min(H, 9)]       # token t = e_t
        lg = moe.router_logits(wr, x)
        assert lg.shape == (x.shape[0], E)
        for t in range(x.shape[0]):
            assert np.array_equal(lg[t], wr[:, t].astype(np.float64))


def test_router_logits_basis_rows_pick_scaled_entries():
    E, H = 12, 64
    pos = np.array([3, 0, 63, 17, 17, 5, 40, 41, 2, 8, 31, 60])
    scale = np.array([1, -2, 0.5, 4, -0.25, 8, 1, -1, 2, 0.125, -4, 16], np.float32)
    wr = np.zeros((E, H), np.float32)
    wr[np.arange(E), pos] = scale
    x = synth.activations(12, 3, H)
    lg = moe.router_logits(wr, x)
    for t in range(3):
        for e in range(E):
            assert lg[t, e] == np.float64(scale[e]) * np.float64(x[t, pos[e]])


def test_router_logits_integer_brute_force():
    rng = np.random.default_rng(13)
    E, H, m = 7, 40, 2
    wr = rng.integers(-50, 51, size=(E, H))
    x = rng.integers(-30, 31, size=(m, H))
    lg = moe.router_logits(wr.astype(np.float32), x.astype(np.float32))
    for t in range(m):
        for e in range(E):
            exact = sum(int(x[t, i]) * int(wr[e, i]) for i in range(H))
            assert lg[t, e] == float(exact)


# ------------------------------------------- expert chains, other quantizers --

def _identity_down_q4_0(hidden, inter):
    """Q4_0 down matrix [hidden x inter] with d = 1, code 9 (value 1) on the
    diagonal and 8 (value 0) elsewhere: W_down = [I; 0] when hidden >= inter."""
    nb = inter // 32
    q = np.full((hidden, inter), 8, np.int64)
    r = np.arange(min(hidden, inter))
    q[r, r] = 9
    return formats.encode("q4_0", {"d": np.ones((hidden, nb)), "q": q.reshape(hidden, nb, 32)})


def _exact_quant(v):
    """Unquantized activations as 'codes' with unit scales (no rounding)."""
    v = np.atleast_2d(np.asarray(v, np.float32))
    return v.astype(np.float64), np.ones((v.shape[0], v.shape[1] // 32), np.float64), None


def _s16_quant(v):
    from oracle.quant import quantize_s16
    return quantize_s16(v)


@pytest.mark.parametrize("quant_name", ["q8", "s16", "exact"])
def test_expert_chain_identity_down_returns_requantized_h(quant_name):
    # With W_down = [I; 0] the expert's output is its own re-quantized h,
    # dequantized, followed by zeros: this pins the down projection's wiring
    # and the re-quantization rule of each variant.
    quant = {"q8": quantize_q8, "s16": _s16_quant, "exact": _exact_quant}[quant_name]
    H, I = 256, 128
    gu = synth.weights("q4_0", 2 * I, H, seed=21)
    dn = _identity_down_q4_0(H, I)
    x = synth.activations(22, 1, H)
    xq, dx, _ = quant(x)
    ch = moe.expert_chain(gu, dn, xq, dx, H, I, quant=quant)
    hh = dequantize_q8(ch["hq"], ch["hd"])
    assert np.array_equal(ch["out"][:, :I], hh)
    assert np.all(ch["out"][:, I:] == 0.0)
    if quant_name == "exact":
        # no rounding anywhere: the output is h itself, as held in fp32
        assert np.array_equal(ch["out"][0, :I], ch["h"][0].astype(np.float32).astype(np.float64))
    else:
        qmax = 127 if quant_name == "q8" else 32767
        # the codes reach the format's full range in every non-zero block
        assert np.abs(ch["hq"]).reshape(-1, 32).max(axis=1).max() == qmax


@pytest.mark.parametrize("quant_name", ["s16", "exact"])
def test_moe_identical_experts_other_quantizers(quant_name):
    # All routed experts identical: the combine returns that expert plus the
    # shared one for any routing (the weights sum to one), under each
    # activation variant.
    quant = {"s16": _s16_quant, "exact": _exact_quant}[quant_name]
    H, I, E, K = 256, 64, 16, 4
    one_gu = synth.weights("q4_0", 2 * I, H, seed=25)
    one_dn = synth.weights("q4_0", H, I, seed=26)
    sh_gu = synth.weights("q4_0", 2 * I, H, seed=27)
    sh_dn = synth.weights("q4_0", H, I, seed=28)
    wr = synth.router_weights(29, E, H)
    x = synth.activations(30, 3, H)
    r = moe.moe_ref(wr, np.tile(one_gu, E), np.tile(one_dn, E), sh_gu, sh_dn, x, H, I, K, quant=quant)
    for t in range(3):
        xq, dx, _ = quant(x[t:t + 1])
        e = moe.expert_chain(one_gu, one_dn, xq, dx, H, I, quant=quant)["out"][0]
        s = moe.expert_chain(sh_gu, sh_dn, xq, dx, H, I, quant=quant)["out"][0]
        assert np.allclose(r["y"][t], e + s, rtol=1e-13, atol=1e-15)


def test_moe_exact_chain_matches_float_product():
    # Unquantized activations: each expert is the plain product of the
    # decoded matrices with x and with silu(g) * u held in fp32, so the layer
    # equals a hand-assembled fp64 chain.
    H, I, E, K = 128, 64, 8, 3
    gu_all, dn_all = synth.moe_experts(31, E, H, I)
    gu_sh, dn_sh = synth.moe_experts(32, 1, H, I)
    wr = synth.router_weights(33, E, H)
    x = synth.activations(34, 2, H)
    r = moe.moe_ref(wr, gu_all, dn_all, gu_sh, dn_sh, x, H, I, K, quant=_exact_quant)
    sz_gu, sz_dn = 2 * I * synth.row_bytes("q4_0", H), H * synth.row_bytes("q4_0", I)

    def chain(g, d, xt):
        wg = formats.values("q4_0", g, 2 * I, H)
        wd = formats.values("q4_0", d, H, I)
        z = wg @ xt.astype(np.float64)
        h = (z[:I] / (1.0 + np.exp(-z[:I])) * z[I:]).astype(np.float32).astype(np.float64)
        return wd @ h

    for t in range(2):
        lg = x[t].astype(np.float64) @ wr.astype(np.float64).T
        order = sorted(range(E), key=lambda j: (-lg[j], j))[:K]
        w = np.exp(lg[order] - lg[order[0]])
        w /= w.sum()
        y = sum(w[i] * chain(gu_all[e * sz_gu:(e + 1) * sz_gu], dn_all[e * sz_dn:(e + 1) * sz_dn], x[t])
                for i, e in enumerate(order))
        y = y + chain(gu_sh, dn_sh, x[t])
        assert np.allclose(r["y"][t], y, rtol=1e-12, atol=1e-14)
