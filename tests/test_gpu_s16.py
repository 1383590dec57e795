"""GPU parity of the 16-bit activation path (qgemv_run_s16 and its checking
exports) against the oracle: the quantizer's codes, scales and sums
bit-exact, the per-sub-block int32 dots bit-exact, the GEMV within the
normwise bound at every supported K (one- and four-row launches, ragged row
counts, full dense-layer size on sampled rows), and the accuracy it exists
for: far closer to the unquantized-activation product than the int8 path."""
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


def test_quantizer_s16_bit_exact():
    x = synth.activations(60, 5, 4096)
    x[0, :32] = 0.0                                   # zero block
    x[1, :10] = [32767.0, 2.5, -2.5, 0.5, -0.5, 1.5, 32766.5, -32766.5, 0.49999997, 3.5]
    x[1, 10:32] = 0.0                                 # unit-scale block: ties visible
    x[2, 32:64] *= 1e-30                              # tiny scales
    x[3, 64:96] *= 1e30                               # huge scales
    xq, dx, sx = qg.debug_quantize_s16(dev(x))
    torch.cuda.synchronize()
    q, d, s = quantize_s16(x)
    assert np.array_equal(host(xq), q)
    assert np.array_equal(host(dx).view(np.int32), d.view(np.int32))
    assert np.array_equal(host(sx), s)


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k"])
@pytest.mark.parametrize("n,k", [(300, 2048), (100, 4096), (33, 6144), (8195, 4096), (64, 8192)])
def test_block_dots_s16_bit_exact(fmt, n, k):
    w = synth.weights(fmt, n, k, seed=61)
    x = synth.activations(62, 1, k)
    q, _, _ = quantize_s16(x)
    g = qg.GEMV(fmt, n, k)
    dots = host(g.block_dots_s16(dev(w), dev(q[0])))
    torch.cuda.synchronize()
    ref = og.block_dots(fmt, w, n, k, q)[0]
    assert np.array_equal(dots.astype(np.int64), ref)


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k"])
@pytest.mark.parametrize("n,k", [(1, 4096), (100, 2048), (4096, 4096), (8195, 4096), (777, 6144), (12288, 8192)])
def test_gemv_s16_parity(fmt, n, k):
    w = synth.weights(fmt, n, k, seed=63)
    x = synth.activations(64, 1, k)
    g = qg.GEMV(fmt, n, k)
    full, y = guarded(torch, n, torch.float32)
    g.run_s16(dev(w), dev(x), y=y)
    torch.cuda.synchronize()
    assert canary_ok(torch, full, n)
    q, d, _ = quantize_s16(x)
    e = normwise(host(y)[None], og.gemv_dequant(fmt, w, n, k, q, d))
    say(f"s16 gemv {fmt} n={n} k={k}: normwise {e:.2e}")
    assert e <= TOL


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k"])
def test_gemv_s16_full_size_sampled_rows(fmt):
    n, k = 24576, 4096
    w = synth.weights(fmt, n, k, seed=65)
    x = synth.activations(66, 1, k)
    g = qg.GEMV(fmt, n, k)
    y = host(g.run_s16(dev(w), dev(x)))
    torch.cuda.synchronize()
    q, d, _ = quantize_s16(x)
    rows = np.unique(np.linspace(0, n - 1, 800).astype(np.int64))
    assert normwise(y[:, rows], og.gemv_rows(fmt, w, n, k, rows, q, d)) <= TOL


def test_s16_is_closer_to_unquantized_activations():
    # The reason for the variant: against the product with the fp32
    # activations themselves (fp64), 16-bit codes err about 256x less than
    # int8 codes.
    n, k = 2048, 4096
    w = synth.weights("q4_k", n, k, seed=67)
    x = synth.activations(68, 1, k)
    g = qg.GEMV("q4_k", n, k)
    wd, xd = dev(w), dev(x)
    y16 = host(g.run_s16(wd, xd))
    y8 = host(g.run(wd, xd))
    torch.cuda.synchronize()
    # W_hat . x in fp64: the oracle's dequantize form with unit scales and the
    # fp32 activations themselves in place of codes.
    wh = og.gemv_dequant("q4_k", w, n, k, x.astype(np.float64).reshape(1, k), np.ones((1, k // 32)))
    e16, e8 = normwise(y16, wh), normwise(y8, wh)
    say(f"error vs unquantized activations: s16 {e16:.2e}, int8 {e8:.2e}")
    assert e16 * 100 < e8


def test_s16_graph_replays_match_eager():
    n, k = 4096, 4096
    w = dev(synth.weights("q4_k", n, k, seed=69))
    g = qg.GEMV("q4_k", n, k)
    ws = g.workspace_s16()
    xs = [dev(synth.activations(70 + i, 1, k)) for i in range(3)]
    eager = [g.run_s16(w, x, ws=ws).clone() for x in xs]
    x_in = xs[0].clone()
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    g.run_s16(w, x_in, y=y, ws=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.run_s16(w, x_in, y=y, ws=ws)
    for rep in range(3):
        for i in (2, 0, 1):
            x_in.copy_(xs[i])
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager[i]), f"replay {rep} input {i}"
            other = g.run_s16(w, xs[(i + 1) % 3], ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(other, eager[(i + 1) % 3])
