"""Pins for the oracle's Q8 activation quantizer.

The rule (32-element blocks, scale = absmax / 127, codes rounded half away
from zero) is fixed by the decode-GEMV workload description; the pins below
check it against closed forms and against an exact-rational reimplementation
that does its own IEEE binary32 rounding (so numpy's fp32 division is not
trusted blindly).
"""
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle.quant import quantize_q8, dequantize_q8


def _block(vals, fill=0.0):
    x = np.full(32, fill, np.float32)
    x[: len(vals)] = np.asarray(vals, np.float32)
    return x[None, :]


def test_ties_round_half_away_from_zero():
    # absmax 127 makes d = 127/127 = 1 exactly, so v = x and the rounding
    # rule is visible directly. np.round (half to even) would give 2, -2, 0, 0.
    x = _block([127.0, 2.5, -2.5, 0.5, -0.5, 1.5, 126.5, -126.5, np.float32(0.49999997), 3.5])
    q, d, s = quantize_q8(x)
    assert d[0, 0] == np.float32(1.0)
    assert list(q[0, :10]) == [127, 3, -3, 1, -1, 2, 127, -127, 0, 4]
    assert s[0, 0] == int(q[0].astype(np.int64).sum())


def test_zero_block():
    q, d, s = quantize_q8(np.zeros((1, 64), np.float32))
    assert np.all(q == 0) and np.all(d == 0) and np.all(s == 0)


def test_negative_zero_and_mixed_zero_blocks():
    x = np.zeros((2, 64), np.float32)
    x[0, :32] = -0.0
    x[1, 40] = -3.0
    q, d, s = quantize_q8(x)
    assert np.all(q[0] == 0) and d[0, 0] == 0
    assert d[1, 0] == 0 and q[1, 40] == -127 and d[1, 1] == np.float32(3.0) / np.float32(127)


@pytest.mark.parametrize("e", [-20, -3, 0, 5, 30])
def test_power_of_two_round_trip(e):
    # x = 2^e * q with max|q| = 127: d = 2^e exactly, codes come back exactly.
    rng = np.random.default_rng(e + 100)
    qi = rng.integers(-127, 128, size=(3, 96))
    qi[:, ::32] = 127 * np.sign(rng.standard_normal((3, 3)))
    x = (qi * 2.0 ** e).astype(np.float32)
    q, d, s = quantize_q8(x)
    assert np.all(d == np.float32(2.0 ** e))
    assert np.array_equal(q.astype(np.int64), qi)
    assert np.array_equal(dequantize_q8(q, d), x.astype(np.float64))


def _fp32_round(r: Fraction) -> Fraction:
    """Round a rational to the nearest IEEE binary32 value, ties to even."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    t = a / ulp
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def _quant_exact(block):
    a = max(abs(Fraction(float(v))) for v in block)
    if a == 0:
        return [0] * 32, Fraction(0)
    d = _fp32_round(a / 127)
    out = []
    for v in block:
        vv = _fp32_round(Fraction(float(v)) / d)
        mag = abs(vv)
        qv = math.floor(mag + Fraction(1, 2))
        qv = min(qv, 127)
        out.append(qv if vv >= 0 else -qv)
    return out, d


def test_brute_force_against_exact_rationals():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    x[1] *= np.float32(1e-3)
    x[2, :32] = rng.integers(-300, 300, 32).astype(np.float32) / np.float32(4)   # many ties
    q, d, s = quantize_q8(x)
    for r in range(4):
        for b in range(4):
            codes, dd = _quant_exact(x[r, 32 * b:32 * b + 32])
            assert Fraction(float(d[r, b])) == dd
            assert list(q[r, 32 * b:32 * b + 32].astype(int)) == codes
            assert s[r, b] == sum(codes)


def test_absmax_element_maps_to_127():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    q, d, s = quantize_q8(x)
    xb = x.reshape(8, 8, 32)
    idx = np.abs(xb).argmax(-1)
    qb = q.reshape(8, 8, 32)
    got = np.take_along_axis(qb, idx[..., None], -1)[..., 0].astype(int)
    assert np.all(np.abs(got) == 127)
    assert np.all(np.abs(q.astype(int)) <= 127)


def test_reconstruction_error_bound():
    # |x - d*q| <= d/2 (plus fp32 rounding of v) for every element.
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 4096)).astype(np.float32)
    q, d, s = quantize_q8(x)
    err = np.abs(x.astype(np.float64) - dequantize_q8(q, d))
    bound = np.repeat(d.astype(np.float64), 32, axis=1) * (0.5 + 1e-6)
    assert np.all(err <= bound)


# ---- 16-bit variant (scale = absmax / 32767, int16 codes) ----

from oracle.quant import quantize_s16  # noqa: E402


def test_s16_ties_round_half_away_from_zero():
    # absmax 32767 makes d = 1 exactly, so v = x.
    x = _block([32767.0, 2.5, -2.5, 0.5, -0.5, 1.5, 32766.5, -32766.5, np.float32(0.49999997), 3.5])
    q, d, s = quantize_s16(x)
    assert q.dtype == np.int16 and d[0, 0] == np.float32(1.0)
    assert list(q[0, :10]) == [32767, 3, -3, 1, -1, 2, 32767, -32767, 0, 4]
    assert s[0, 0] == int(q[0].astype(np.int64).sum())


@pytest.mark.parametrize("e", [-20, 0, 7])
def test_s16_power_of_two_round_trip(e):
    rng = np.random.default_rng(e + 300)
    qi = rng.integers(-32767, 32768, size=(2, 64))
    qi[:, ::32] = 32767
    x = (qi * 2.0 ** e).astype(np.float32)
    q, d, s = quantize_s16(x)
    assert np.all(d == np.float32(2.0 ** e))
    assert np.array_equal(q.astype(np.int64), qi)
    assert np.array_equal(s.astype(np.int64), qi.reshape(2, 2, 32).sum(-1))


def test_s16_zero_block_and_exact_rationals():
    q, d, s = quantize_s16(np.zeros((1, 32), np.float32))
    assert np.all(q == 0) and d[0, 0] == 0 and s[0, 0] == 0
    # The exact-rational restatement above (binary32 rounding of the scale
    # and of every quotient), with 32767 in place of 127.
    rng = np.random.default_rng(7)
    for _ in range(20):
        x = (rng.standard_normal(32) * 10.0 ** rng.integers(-3, 4)).astype(np.float32)
        q, d, s = quantize_s16(x[None])
        a = max(abs(Fraction(float(v))) for v in x)
        dd = _fp32_round(a / 32767)
        assert Fraction(float(d[0, 0])) == dd
        for i, v in enumerate(x):
            t = _fp32_round(Fraction(float(v)) / dd) if v != 0 else Fraction(0)
            want = int(math.copysign(math.floor(abs(t) + Fraction(1, 2)), t))
            want = max(-32767, min(32767, want))
            assert int(q[0, i]) == want


def test_s16_step_is_256_times_finer_and_error_bound():
    # The page's ledger reports a 256x smaller quantization step: the scale
    # ratio is 127 / 32767 (about 1/258), and |x - d q| <= d / 2 holds.
    x = np.random.default_rng(8).standard_normal((4, 256)).astype(np.float32)
    q8, d8, _ = quantize_q8(x)
    q16, d16, _ = quantize_s16(x)
    ratio = d8.astype(np.float64) / d16.astype(np.float64)
    assert np.allclose(ratio, 32767 / 127, rtol=1e-6)
    err = np.abs(x.astype(np.float64) - dequantize_q8(q16, d16))
    assert np.all(err <= np.repeat(d16.astype(np.float64), 32, axis=1) / 2 * (1 + 1e-6))
    err8 = np.abs(x.astype(np.float64) - dequantize_q8(q8, d8))
    assert err.max() * 200 < err8.max()
