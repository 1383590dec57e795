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
