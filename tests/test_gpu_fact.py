"""GPU parity of the float-activation batched GEMV (qgemv_run_f32act) against
the oracle's float-activation form: within the normwise bound for Q4_0 and
Q8_0 over ragged row counts, K below one block per wave, 1..32 tokens (one
and two token tiles) and the full dense-layer size; no write outside y;
repeat calls and graph replays bit-identical to eager calls; and the accuracy
it exists for: far closer to the unquantized-activation product than the int8
path."""
import numpy as np
import pytest

import synth
from oracle import gemv as og
from tests.gpu_util import TOL, canary_ok, dev, guarded, host, normwise, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import block_quant_gemv_amd as qg  # noqa: E402


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("n,k,m", [(1, 32, 1), (37, 96, 3), (300, 1024, 16), (300, 1024, 17),
                                   (1000, 2048, 32), (4095, 512, 9), (16, 4096, 2), (129, 8192, 31),
                                   (517, 2048, 5), (300, 4096, 8), (33, 1024, 7)])
def test_f32act_parity(fmt, n, k, m):
    say(f"f32act parity {fmt} n={n} k={k} m={m}")
    w = synth.weights(fmt, n, k, seed=71)
    x = synth.activations(72, m, k)
    g = qg.GEMV(fmt, n, k, max_m=32)
    full, y = guarded(torch, m * n, torch.float32)
    g.run_f32act(dev(w), dev(x), y=y.view(m, n))
    torch.cuda.synchronize()
    assert canary_ok(torch, full, m * n)
    ref = og.gemv_float_act(fmt, w, n, k, x)
    err = normwise(host(y).reshape(m, n), ref)
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("m", [1, 32])
def test_f32act_full_size(fmt, m):
    n = k = 4096
    say(f"f32act full size {fmt} {n}x{k} m={m}")
    w = synth.weights(fmt, n, k, seed=73)
    x = synth.activations(74, m, k)
    g = qg.GEMV(fmt, n, k, max_m=32)
    wd, xd = dev(w), dev(x)
    y1 = host(g.run_f32act(wd, xd))
    y2 = host(g.run_f32act(wd, xd))
    torch.cuda.synchronize()
    assert np.array_equal(y1.view(np.int32), y2.view(np.int32))  # fixed summation order
    err = normwise(y1, og.gemv_float_act(fmt, w, n, k, x))
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_f32act_more_accurate_than_int8(fmt):
    n, k, m = 512, 4096, 8
    w = synth.weights(fmt, n, k, seed=75)
    x = synth.activations(76, m, k)
    g = qg.GEMV(fmt, n, k, max_m=32)
    yf = host(g.run_f32act(dev(w), dev(x)))
    yq = host(g.run(dev(w), dev(x)))
    torch.cuda.synchronize()
    truth = og.gemv_float_act(fmt, w, n, k, x)
    ef, eq = normwise(yf, truth), normwise(yq, truth)
    say(f"{fmt}: float activations {ef:.2e}, int8 activations {eq:.2e}")
    assert ef * 100 < eq


def test_f32act_graph_replays_match_eager():
    n, k, m = 4096, 4096, 24
    w = dev(synth.weights("q8_0", n, k, seed=77))
    g = qg.GEMV("q8_0", n, k, max_m=32)
    xs = [dev(synth.activations(78 + i, m, k)) for i in range(3)]
    eager = [g.run_f32act(w, x).clone() for x in xs]
    x_in = xs[0].clone()
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    g.run_f32act(w, x_in, y=y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.run_f32act(w, x_in, y=y)
    for rep in range(3):
        for i in (2, 0, 1):
            x_in.copy_(xs[i])
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager[i]), f"replay {rep} input {i}"
            other = g.run_f32act(w, xs[(i + 1) % 3])
            torch.cuda.synchronize()
            assert torch.equal(other, eager[(i + 1) % 3])
