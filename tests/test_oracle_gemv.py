"""Pins for the oracle's GEMV: two independent forms, exact rationals, and the
unit-scale special case that reduces to an integer matmul."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats, gemv
from oracle.quant import quantize_q8

FMTS = formats.FORMATS


def _cb():
    return synth.codebook(9)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 3])
def test_intdot_form_equals_dequant_form(fmt, m):
    n, k = 37, 1024
    raw = synth.weights(fmt, n, k, seed=4)
    x = synth.activations(5, m, k)
    cb = _cb()
    xq, dx, sx = quantize_q8(x)
    y2 = gemv.gemv_dequant(fmt, raw, n, k, xq, dx, cb)
    y1 = gemv.gemv_intdot(fmt, raw, n, k, xq, dx, sx, cb)
    assert np.linalg.norm(y1 - y2) <= 1e-13 * np.linalg.norm(y2)


@pytest.mark.parametrize("fmt", FMTS)
def test_unit_scales_reduce_to_integer_matmul(fmt):
    # d = 1, sc = 1, m = 0, dmin = 0 and activations with block absmax 127
    # (so dx = 1, xq = x): y must equal the int64 matmul of the code matrices.
    n, k = 9, 512
    rng = np.random.default_rng(21)
    nb = k // formats.BLOCK_ELEMS[fmt]
    f = {"d": np.ones((n, nb))}
    cb = _cb().astype(np.int64)
    if fmt in ("q4_0", "iq4_nl"):
        f["q"] = rng.integers(0, 16, (n, nb, 32))
        ints = (f["q"] - 8) if fmt == "q4_0" else cb[f["q"]]
    elif fmt == "q8_0":
        f["q"] = rng.integers(-127, 128, (n, nb, 32))
        ints = f["q"]
    elif fmt in ("q4_k", "q5_k"):
        top = 16 if fmt == "q4_k" else 32
        f.update(dmin=np.zeros((n, nb)), sc=np.ones((n, nb, 8), np.int64),
                 m=np.zeros((n, nb, 8), np.int64), q=rng.integers(0, top, (n, nb, 256)))
        ints = f["q"]
    elif fmt == "iq4_xs":
        f.update(ls=np.full((n, nb, 8), 33, np.int64), q=rng.integers(0, 16, (n, nb, 256)))
        ints = cb[f["q"]]
    else:
        f.update(sc=np.ones((n, nb, 16), np.int64), q=rng.integers(0, 64, (n, nb, 256)))
        ints = f["q"] - 32
    W = ints.reshape(n, k)
    raw = formats.encode(fmt, f)
    xi = rng.integers(-127, 128, (2, k))
    xi[:, ::32] = 127
    xq, dx, sx = quantize_q8(xi.astype(np.float32))
    assert np.all(dx == 1) and np.array_equal(xq.astype(np.int64), xi)
    expect = xi @ W.T
    y = gemv.gemv_dequant(fmt, raw, n, k, xq, dx, cb)
    assert np.array_equal(y, expect.astype(np.float64))
    yi = gemv.gemv_intdot(fmt, raw, n, k, xq, dx, sx, cb)
    assert np.array_equal(yi, expect.astype(np.float64))


@pytest.mark.parametrize("fmt", FMTS)
def test_block_dots_equal_naive_python_sums(fmt):
    n, k = 3, 512
    raw = synth.weights(fmt, n, k, seed=6)
    x = synth.activations(8, 2, k)
    xq, _, _ = quantize_q8(x)
    cb = _cb()
    D = gemv.block_dots(fmt, raw, n, k, xq, cb)
    f = formats.decode(fmt, raw, n, k)
    q = f["q"].reshape(n, k)
    g = 16 if fmt == "q6_k" else 32
    for t in range(2):
        for r in range(n):
            for b in range(k // g):
                acc = 0
                for i in range(b * g, b * g + g):
                    c = int(q[r, i])
                    if fmt == "q4_0":
                        c -= 8
                    elif fmt in ("iq4_nl", "iq4_xs"):
                        c = int(cb[c])
                    elif fmt == "q6_k":
                        c -= 32
                    acc += int(xq[t, i]) * c
                assert D[t, r, b] == acc
    assert np.abs(D).max() <= 32 * 127 * 127


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [32, 64, 256])
def test_exact_rationals_tiny(fmt, k):
    if k % formats.BLOCK_ELEMS[fmt]:
        pytest.skip("K below the super-block size")
    n = 4
    raw = synth.weights(fmt, n, k, seed=k)
    x = synth.activations(k + 1, 1, k)
    xq, dx, sx = quantize_q8(x)
    cb = _cb()
    y = gemv.gemv_dequant(fmt, raw, n, k, xq, dx, cb)[0]
    w = formats.values(fmt, raw, n, k, cb)
    for r in range(n):
        exact = sum(Fraction(float(w[r, i])) * Fraction(float(dx[0, i // 32])) * int(xq[0, i])
                    for i in range(k))
        scale = sum(abs(Fraction(float(w[r, i])) * Fraction(float(dx[0, i // 32])) * int(xq[0, i]))
                    for i in range(k))
        assert abs(Fraction(float(y[r])) - exact) <= Fraction(1, 2 ** 50) * (scale + 1)


def test_scale_linearity_q4_0():
    n, k = 8, 256
    rng = np.random.default_rng(2)
    q = rng.integers(0, 16, (n, k // 32, 32))
    d = rng.uniform(1e-3, 1e-2, (n, k // 32)).astype(np.float16).astype(np.float64)
    r1 = formats.encode("q4_0", {"d": d, "q": q})
    r2 = formats.encode("q4_0", {"d": 2 * d, "q": q})
    x = synth.activations(3, 1, k)
    xq, dx, _ = quantize_q8(x)
    y1 = gemv.gemv_dequant("q4_0", r1, n, k, xq, dx)
    y2 = gemv.gemv_dequant("q4_0", r2, n, k, xq, dx)
    assert np.array_equal(2 * y1, y2)


def test_rows_subset_matches_full():
    n, k = 300, 512
    raw = synth.weights("q6_k", n, k, seed=1)
    x = synth.activations(2, 1, k)
    xq, dx, _ = quantize_q8(x)
    full = gemv.gemv_dequant("q6_k", raw, n, k, xq, dx)
    rows = np.array([0, 7, 150, 299])
    sub = gemv.gemv_rows("q6_k", raw, n, k, rows, xq, dx)
    assert np.array_equal(sub, full[:, rows])


def test_iq4_xs_sub_scales_scale_each_sub_block():
    # Changing one sub-scale changes only that sub-block's share of y, by the
    # ratio of (ls - 32): y is linear in each sub-block's scale.
    n, k = 3, 512
    rng = np.random.default_rng(31)
    nb = k // 256
    cb = _cb()
    q = rng.integers(0, 16, (n, nb, 256))
    d = np.full((n, nb), 0.25)
    ls = rng.integers(0, 64, (n, nb, 8))
    ls[:, 1, 5] = 40
    base = formats.encode("iq4_xs", {"d": d, "ls": ls, "q": q})
    ls2 = ls.copy()
    ls2[:, 1, 5] = 48
    other = formats.encode("iq4_xs", {"d": d, "ls": ls2, "q": q})
    x = synth.activations(4, 1, k)
    xq, dx, _ = quantize_q8(x)
    y1 = gemv.gemv_dequant("iq4_xs", base, n, k, xq, dx, cb)
    y2 = gemv.gemv_dequant("iq4_xs", other, n, k, xq, dx, cb)
    # the affected sub-block covers elements 256 + 160 .. 256 + 191
    sl = slice(256 + 160, 256 + 192)
    part = (dx[0, sl.start // 32] * xq[0, sl].astype(np.float64)) @ (0.25 * cb[q[:, 1, 160:192]].T)
    assert np.allclose(y2 - y1, (48 - 32 - (40 - 32)) * part, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", FMTS)
def test_float_act_equals_quantized_form_on_the_q8_grid(fmt):
    # Activations that Q8 quantization reproduces exactly (codes with a +-127
    # in every block, power-of-two block scales): the float-activation form
    # and the quantized dequantize form must then give the same products.
    n, m, k = 23, 3, 512
    rng = np.random.default_rng(31)
    raw = synth.weights(fmt, n, k, seed=6)
    cb = _cb()
    q = rng.integers(-127, 128, size=(m, k // 32, 32))
    q[..., 0] = np.where(rng.random((m, k // 32)) < 0.5, 127, -127)
    dx = np.exp2(rng.integers(-6, 3, size=(m, k // 32))).astype(np.float32)
    x = (q * dx[..., None]).reshape(m, k).astype(np.float32)
    xq, dx2, _ = quantize_q8(x)
    assert np.array_equal(xq.astype(np.int64), q.reshape(m, k)) and np.array_equal(dx2, dx)
    yf = gemv.gemv_float_act(fmt, raw, n, k, x, cb)
    yq = gemv.gemv_dequant(fmt, raw, n, k, xq, dx2, cb)
    assert np.linalg.norm(yf - yq) <= 1e-13 * np.linalg.norm(yq)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_float_act_one_hot_inputs_pick_weight_columns(fmt):
    # x = e_j (token 0) and 2 e_j (token 1): y[t, r] = (t + 1) W_hat[r, j], with
    # W_hat[r, j] = d * code from the stored bytes, read here directly.
    n, k = 5, 64
    raw = synth.weights(fmt, n, k, seed=8)
    bb = formats.BLOCK_BYTES[fmt]
    rb = formats.row_bytes(fmt, k)
    rows = np.asarray(raw, np.uint8)[: n * rb].reshape(n, rb)[:, : (k // 32) * bb].reshape(n, k // 32, bb)
    for j in (0, 17, 33, 63):
        x = np.zeros((2, k), np.float32)
        x[0, j], x[1, j] = 1.0, 2.0
        y = gemv.gemv_float_act(fmt, raw, n, k, x)
        b, e = divmod(j, 32)
        d = rows[:, b, 0:2].copy().view(np.float16).astype(np.float64)[:, 0]
        if fmt == "q8_0":
            code = rows[:, b, 2 + e].astype(np.int8).astype(np.float64)
        else:
            byte = rows[:, b, 2 + (e % 16)]
            code = ((byte & 0xF) if e < 16 else (byte >> 4)).astype(np.float64) - 8
        assert np.array_equal(y[0], d * code) and np.array_equal(y[1], 2 * d * code)
