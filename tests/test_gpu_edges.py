"""GPU parity at the edges of the block formats, and on every output row of
the largest workload shapes.

Edges the random workload inputs never produce but the formats allow:
* Q8_0 codes of -128 (the int8 field's one value outside -127..127);
* Q6_K sub-scales of -128 and 127 (the int8 field's ends, outside the
  workloads' -64..63), which push the integer combination sc_a*P0 + sc_b*P1
  to its largest magnitude;
* fp16 block scales at both ends of the format: subnormals (the smallest,
  2^-24, and the largest, just below 2^-14), the smallest normal and 65504,
  for d and for the K-quants' dmin.
Each runs through every device path that reads the format: the decode GEMV
(one and several tokens, fused and separate quantizer), the register-direct
single-token K-quant kernel, the int8 matrix-core batched kernel, the
float-activation kernel and the 16-bit-activation kernel. Per-block integer
dots must equal the oracle's exactly and outputs must be within the normwise
bound.

Full size: the IQ4_NL lm_head (248320 rows) and the N=24576 dense-layer
matrices are compared on every row, and their block dots in full.
"""
import numpy as np
import pytest

import synth
from oracle import gemv as og
from oracle.quant import quantize_q8, quantize_s16
from tests.gpu_util import TOL, canary_ok, dev, guarded, host, normwise, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import block_quant_gemv_amd as qg  # noqa: E402

CB = synth.codebook(77)
CB_FORMATS = ("iq4_nl", "iq4_xs")

# fp16 bit patterns: smallest subnormal, largest subnormal, smallest normal,
# largest finite, and one ordinary value
F16_EDGES = np.array([0x0001, 0x03FF, 0x0400, 0x7BFF, 0x2000], np.uint16)


def _blocks(raw, fmt, n, k):
    bb = synth.BLOCK_BYTES[fmt]
    nb = synth.row_bytes(fmt, k) // bb
    return raw[: n * nb * bb].reshape(n, nb, bb)


def _plant(fmt, n, k, seed, *, q8_min=False, q6_ext=False, f16_ext=False):
    """Workload-style weights with edge values planted at seeded positions."""
    raw = synth.weights(fmt, n, k, seed=seed)
    blk = _blocks(raw, fmt, n, k)
    rng = np.random.default_rng(seed + 1)
    if q8_min:
        codes = blk[..., 2:34]
        codes[rng.random(codes.shape) < 0.15] = 0x80       # int8 -128
        blk[0, 0, 2:34] = 0x80                              # one block entirely -128
    if q6_ext:
        sc = blk[..., 2:18]
        pick = rng.integers(0, 4, size=sc.shape)
        vals = np.array([-128, 127, -64, 63], np.int8).view(np.uint8)
        mask = rng.random(sc.shape) < 0.5
        sc[mask] = vals[pick[mask]]
        blk[0, 0, 2:18] = np.array([-128] * 8 + [127] * 8, np.int8).view(np.uint8)
    if f16_ext:
        offs = [0, 2] if fmt in ("q4_k", "q5_k") else [0]
        for off in offs:
            pat = F16_EDGES[rng.integers(0, F16_EDGES.size, size=blk.shape[:2])]
            blk[..., off:off + 2] = pat.astype("<u2").view(np.uint8).reshape(*blk.shape[:2], 2)
    return raw


def _check_int8_path(fmt, w, n, k, m, seed, label):
    cb = CB if fmt in CB_FORMATS else None
    x = synth.activations(seed, m, k)
    g = qg.GEMV(fmt, n, k, max_m=m, codebook=cb)
    wd = dev(w)
    full, y = guarded(torch, m * n, torch.float32)
    g.run(wd, dev(x), y.view(m, n))
    xq, dx, _ = quantize_q8(x)
    dots = host(g.block_dots(wd, dev(xq)))
    torch.cuda.synchronize()
    assert canary_ok(torch, full, m * n)
    ref_dots = og.block_dots(fmt, w, n, k, xq, cb)
    bad = np.argwhere(dots != ref_dots)
    assert bad.size == 0, f"{label}: {len(bad)} block dots differ, first {bad[:3].tolist()}"
    ref = og.gemv_dequant(fmt, w, n, k, xq, dx, cb)
    yy = host(y).reshape(m, n)
    assert np.all(np.isfinite(yy))
    e = normwise(yy, ref)
    say(f"  {label}: normwise error {e:.3e}")
    assert e <= TOL


# ---------------------------------------------------- Q8_0 codes of -128 --

@pytest.mark.parametrize("n,k,m", [(1000, 2048, 1),    # fused quantizer
                                   (4096, 4096, 1),    # separate quantizer, K-segmented steps
                                   (300, 4096, 5),     # several tokens
                                   (257, 288, 16)])
def test_q8_0_code_minus_128(n, k, m):
    say(f"q8_0 with -128 codes n={n} k={k} m={m}")
    w = _plant("q8_0", n, k, seed=500 + m, q8_min=True)
    assert (_blocks(w, "q8_0", n, k)[..., 2:34] == 0x80).mean() > 0.1
    _check_int8_path("q8_0", w, n, k, m, seed=510 + m, label="q8_0 -128")


@pytest.mark.parametrize("m", [1, 32])
def test_q8_0_code_minus_128_float_activations(m):
    n, k = 700, 4096
    say(f"q8_0 -128 codes, float activations m={m}")
    w = _plant("q8_0", n, k, seed=520, q8_min=True)
    x = synth.activations(521, m, k)
    g = qg.GEMV("q8_0", n, k, max_m=32)
    y = host(g.run_f32act(dev(w), dev(x)))
    torch.cuda.synchronize()
    e = normwise(y, og.gemv_float_act("q8_0", w, n, k, x))
    say(f"  normwise error {e:.3e}")
    assert e <= TOL


# ------------------------------------------- Q6_K sub-scales of -128, 127 --

@pytest.mark.parametrize("n,k,m", [(4096, 12288, 1),   # FFN down shape
                                   (300, 2048, 3),     # several tokens, fused quantizer
                                   (64, 512, 9),       # int8 matrix cores from 9 tokens
                                   (1024, 12288, 32)])  # batched shape tile, K split
def test_q6_k_extreme_subscales(n, k, m):
    say(f"q6_k with sub-scales -128/127 n={n} k={k} m={m}")
    w = _plant("q6_k", n, k, seed=530 + m, q6_ext=True)
    sc = _blocks(w, "q6_k", n, k)[..., 2:18].view(np.int8)
    assert (sc == -128).any() and (sc == 127).any()
    _check_int8_path("q6_k", w, n, k, m, seed=540 + m, label="q6_k extreme sc")


# ------------------------------------------------- fp16 scales at the ends --

F16_CASES = [
    ("q4_0", 2048, 2048, 1), ("q8_0", 4096, 4096, 1), ("iq4_nl", 1500, 4096, 1),
    ("q4_k", 4096, 4096, 1),      # register-direct kernel (d and dmin)
    ("q5_k", 2048, 4096, 1),      # register-direct kernel
    ("q4_k", 500, 4096, 3),       # decode GEMV, several tokens
    ("q6_k", 4096, 12288, 1), ("iq4_xs", 1000, 4096, 2),
    ("q4_k", 1000, 4096, 32),     # int8 matrix cores
    ("q6_k", 500, 4096, 17),
]


@pytest.mark.parametrize("fmt,n,k,m", F16_CASES)
def test_fp16_scale_extremes(fmt, n, k, m):
    say(f"{fmt} with fp16 scales at the ends n={n} k={k} m={m}")
    w = _plant(fmt, n, k, seed=550 + n % 97, f16_ext=True)
    _check_int8_path(fmt, w, n, k, m, seed=560 + m, label=f"{fmt} fp16 ends")


@pytest.mark.parametrize("fmt,m", [("q4_0", 1), ("q8_0", 32), ("q4_0", 20)])
def test_fp16_scale_extremes_float_activations(fmt, m):
    n, k = 600, 2048
    say(f"{fmt} fp16 ends, float activations m={m}")
    w = _plant(fmt, n, k, seed=570, f16_ext=True)
    x = synth.activations(571, m, k)
    g = qg.GEMV(fmt, n, k, max_m=32)
    y = host(g.run_f32act(dev(w), dev(x)))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(y))
    e = normwise(y, og.gemv_float_act(fmt, w, n, k, x))
    say(f"  normwise error {e:.3e}")
    assert e <= TOL


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k"])
def test_fp16_scale_extremes_16bit_activations(fmt):
    n, k = 2000, 4096
    say(f"{fmt} fp16 ends, 16-bit activations")
    w = _plant(fmt, n, k, seed=580, f16_ext=True)
    x = synth.activations(581, 1, k)
    g = qg.GEMV(fmt, n, k)
    y = host(g.run_s16(dev(w), dev(x)))
    torch.cuda.synchronize()
    xq, dx, _ = quantize_s16(x)
    e = normwise(y, og.gemv_dequant(fmt, w, n, k, xq, dx))
    say(f"  normwise error {e:.3e}")
    assert e <= TOL


# ------------------------------------------------------ full size, all rows --

@pytest.mark.parametrize("fmt,n", [("q8_0", 24576), ("q4_k", 24576), ("iq4_nl", 248320)])
def test_full_size_every_row_and_block_dots(fmt, n):
    k = 4096
    say(f"full size {fmt} n={n} k={k}: every output row and every block dot")
    cb = CB if fmt in CB_FORMATS else None
    w = synth.weights(fmt, n, k, seed=590)
    x = synth.activations(591, 1, k)
    g = qg.GEMV(fmt, n, k, codebook=cb)
    wd = dev(w)
    y = host(g.run(wd, dev(x)))
    xq, dx, _ = quantize_q8(x)
    dots = host(g.block_dots(wd, dev(xq)))
    torch.cuda.synchronize()
    del wd
    ref_dots = og.block_dots(fmt, w, n, k, xq, cb)
    bad = np.argwhere(dots != ref_dots)
    assert bad.size == 0, f"{len(bad)} block dots differ, first {bad[:3].tolist()}"
    del dots, ref_dots
    ref = og.gemv_dequant(fmt, w, n, k, xq, dx, cb)
    e = normwise(y, ref)
    rowrel = np.abs(y - ref) / (np.abs(ref) + np.abs(ref).mean())
    say(f"  normwise error {e:.3e}, max per-row relative {rowrel.max():.2e}")
    assert e <= TOL
    assert rowrel.max() <= 1e-4


# --------------------------------------------------------- codebooks --
# The device looks a code up in two byte-permute pools that the library
# derives from the codebook; the pools depend on the signs of the entries.
# Codebooks of every sign pattern: all negative, all non-negative, the int8
# ends -128 and 127, sign change at each position of the first half, and
# random ones.
def _codebooks():
    out = [np.arange(-128, -112, dtype=np.int8), np.arange(0, 16, dtype=np.int8),
           np.array([-128, -127] + list(range(-5, 8)) + [127], np.int8)]
    for neg in (1, 3, 5, 7, 9, 12, 15):
        out.append(np.array(list(range(-neg, 0)) + list(range(1, 17 - neg)), np.int8))
    out += [synth.codebook(s) for s in (1, 2, 3)]
    return out


@pytest.mark.parametrize("fmt", CB_FORMATS)
def test_codebook_sign_patterns(fmt):
    n, k, m = 96, 512, 2
    w = synth.weights(fmt, n, k, seed=31)
    x = synth.activations(32, m, k)
    xq, dx, _ = quantize_q8(x)
    for i, cb in enumerate(_codebooks()):
        say(f"codebook {i} {fmt}: {cb.tolist()}")
        assert np.all(np.diff(cb.astype(np.int32)) > 0)
        g = qg.GEMV(fmt, n, k, max_m=m, codebook=cb)
        wd = dev(w)
        y = torch.empty(m, n, dtype=torch.float32, device="cuda")
        g.run(wd, dev(x), y)
        dots = g.block_dots(wd, dev(xq))
        torch.cuda.synchronize()
        ref_dots = og.block_dots(fmt, w, n, k, xq, cb)
        bad = np.argwhere(host(dots) != ref_dots)
        assert bad.size == 0, f"codebook {i}: {len(bad)} block dots differ, first {bad[:3].tolist()}"
        assert normwise(host(y), og.gemv_dequant(fmt, w, n, k, xq, dx, cb)) <= TOL


# One token through the register-direct K-quant kernel (Q5_K, IQ4_XS): K of
# 2048 / 4096 / 8192 (one to four sub-blocks per lane), row counts that leave
# a ragged last group of rows (groups of 2 or 4 rows from 8192 rows), and for
# IQ4_XS codebooks of different sign patterns. Block dots exact, outputs
# within the normwise bound.
@pytest.mark.parametrize("fmt,n,k", [("iq4_xs", 8195, 2048), ("iq4_xs", 37, 8192), ("iq4_xs", 8193, 4096),
                                     ("q5_k", 8195, 2048), ("q5_k", 8194, 8192), ("q5_k", 37, 4096)])
def test_register_direct_one_token(fmt, n, k):
    cbs = [CB, np.arange(-128, -112, dtype=np.int8)] if fmt == "iq4_xs" else [None]
    w = synth.weights(fmt, n, k, seed=n + k)
    x = synth.activations(n + 1, 1, k)
    xq, dx, _ = quantize_q8(x)
    wd = dev(w)
    for cb in cbs:
        say(f"register-direct {fmt} n={n} k={k} codebook={None if cb is None else int(cb[0])}")
        g = qg.GEMV(fmt, n, k, codebook=cb)
        full, y = guarded(torch, n, torch.float32)
        g.run(wd, dev(x), y.view(1, n))
        dots = g.block_dots(wd, dev(xq))
        torch.cuda.synchronize()
        assert canary_ok(torch, full, n), "output guard band overwritten"
        ref_dots = og.block_dots(fmt, w, n, k, xq, cb)
        bad = np.argwhere(host(dots) != ref_dots)
        assert bad.size == 0, f"{len(bad)} block dots differ, first {bad[:3].tolist()}"
        e = normwise(host(y).reshape(1, n), og.gemv_dequant(fmt, w, n, k, xq, dx, cb))
        say(f"  normwise error {e:.3e}")
        assert e <= TOL
