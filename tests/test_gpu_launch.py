"""First launches at awkward moments: inside HIP graph capture, and from
several host threads at once.

The library caches per-device launch facts (compute units, resident
workgroups per kernel, raised LDS limits) on first use of each kernel. The
tests clear that cache so that a fresh plan's very first call happens where
the test wants it, then check the results bit for bit against eager calls
made afterwards and against the oracle."""
import threading

import numpy as np
import pytest

import synth
from oracle import gemv as og
from oracle.quant import quantize_q8
from tests.gpu_util import TOL, dev, host, normwise, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import block_quant_gemv_amd as qg  # noqa: E402


@pytest.mark.parametrize("fmt,n,k,m", [("q8_0", 4096, 4096, 1),    # separate quantizer + GEMV
                                       ("q4_0", 2048, 2048, 1),    # quantizer fused into the GEMV
                                       ("q4_k", 3000, 4096, 1),    # register-direct kernel
                                       ("q6_k", 1000, 4096, 32)])  # int8 matrix cores + split reduce
def test_first_call_of_fresh_plan_inside_capture(fmt, n, k, m):
    say(f"first call inside capture: {fmt} n={n} k={k} m={m}")
    w = synth.weights(fmt, n, k, seed=800)
    xs = [synth.activations(801 + i, m, k) for i in range(2)]
    wd = dev(w)
    x_in = dev(xs[0])
    y_out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    qg.clear_launch_cache()
    g = qg.GEMV(fmt, n, k, max_m=m)
    ws = g.workspace(m)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.run(wd, x_in, y=y_out, ws=ws)       # the plan's (and kernels') first call
    torch.cuda.synchronize()
    eager = []
    for i in range(2):
        eager.append(g.run(wd, dev(xs[i])).clone())
    torch.cuda.synchronize()
    for rep in range(3):
        for i in (1, 0):
            x_in.copy_(dev(xs[i]))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_out, eager[i]), f"replay {rep} input {i}"
    xq, dx, _ = quantize_q8(xs[0])
    assert normwise(host(eager[0]), og.gemv_dequant(fmt, w, n, k, xq, dx)) <= TOL


def test_first_call_of_fresh_ffn_inside_capture():
    H, I = 1024, 2048
    wgu = synth.weights("q4_k", 2 * I, H, seed=810)
    wdn = synth.weights("q6_k", H, I, seed=811)
    x = dev(synth.activations(812, 1, H))
    gu_d, dn_d = dev(wgu), dev(wdn)
    y_out = torch.empty((1, H), dtype=torch.float32, device="cuda")
    qg.clear_launch_cache()
    f = qg.FFN(H, I)
    ws = f.workspace(1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f.run(gu_d, dn_d, x, y=y_out, ws=ws)
    graph.replay()
    torch.cuda.synchronize()
    first = y_out.clone()
    eager = f.run(gu_d, dn_d, x).clone()
    torch.cuda.synchronize()
    assert torch.equal(first, eager)


def test_first_calls_from_several_threads():
    # Eight plans, each first used from its own thread on its own stream at
    # the same moment (ctypes releases the GIL for the library call, so the
    # host code really runs concurrently); every result must equal a later
    # single-threaded call bit for bit.
    cases = [("q8_0", 4096, 4096, 1), ("q4_k", 4100, 4096, 1), ("q6_k", 2000, 12288, 1),
             ("iq4_nl", 3000, 4096, 1), ("q4_0", 2048, 2048, 1), ("q4_k", 600, 4096, 32),
             ("q8_0", 900, 4096, 5), ("q5_k", 1000, 4096, 1)]
    ws_ = [synth.weights(f, n, k, seed=820 + i) for i, (f, n, k, m) in enumerate(cases)]
    xs_ = [synth.activations(830 + i, m, k) for i, (f, n, k, m) in enumerate(cases)]
    wd = [dev(w) for w in ws_]
    xd = [dev(x) for x in xs_]
    plans = [qg.GEMV(f, n, k, max_m=m, codebook=synth.codebook(77) if f == "iq4_nl" else None)
             for f, n, k, m in cases]
    wss = [p.workspace(m) for p, (_, _, _, m) in zip(plans, cases)]
    ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for _, n, _, m in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    qg.clear_launch_cache()
    barrier = threading.Barrier(len(cases))
    errors = []

    def work(i):
        try:
            torch.cuda.set_device(0)
            barrier.wait()
            with torch.cuda.stream(streams[i]):
                plans[i].run(wd[i], xd[i], y=ys[i], ws=wss[i], stream=streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (f, n, k, m) in enumerate(cases):
        again = plans[i].run(wd[i], xd[i])
        torch.cuda.synchronize()
        say(f"  thread {i}: {f} n={n} k={k} m={m}")
        assert torch.equal(ys[i], again), f"case {i} differs from the single-threaded call"
        xq, dx, _ = quantize_q8(xs_[i])
        cb = synth.codebook(77) if f == "iq4_nl" else None
        rows = np.unique(np.linspace(0, n - 1, min(n, 400)).astype(np.int64))
        ref = og.gemv_rows(f, ws_[i], n, k, rows, xq, dx, cb)
        assert normwise(host(again)[:, rows], ref) <= TOL
