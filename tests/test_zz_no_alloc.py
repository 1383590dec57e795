"""The allocation-free GEMV entry point (qgemv_run_noalloc) against
qgemv_run with a caller-allocated workspace: the same kernels, so the same
bits, on two calls in a row where the second has a smaller input, across the
decode, fused-quantizer, register-direct and matrix-core paths; and its size
limit, reported as an error."""
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

# (fmt, n, k, max_m, first m, second m): the second call of each pair is smaller
PAIRS = [
    ("q8_0", 4096, 4096, 8, 8, 1),      # separate quantizer + decode GEMV
    ("q4_0", 2048, 2048, 4, 3, 1),      # quantizer fused into the GEMV
    ("q4_k", 12288, 4096, 32, 32, 1),   # int8 matrix cores, then register-direct
    ("q6_k", 1024, 12288, 32, 32, 9),   # matrix cores, K split over 8 waves
]


@pytest.mark.parametrize("fmt,n,k,max_m,m1,m2", PAIRS)
def test_noalloc_matches_run_two_calls(fmt, n, k, max_m, m1, m2):
    w = dev(synth.weights(fmt, n, k, seed=900))
    g = qg.GEMV(fmt, n, k, max_m=max_m)
    for call, m in enumerate((m1, m2)):
        say(f"noalloc {fmt} n={n} k={k} call {call} m={m}")
        x_np = synth.activations(901 + call, m, k)
        x = dev(x_np)
        y_na = g.run_noalloc(w, x)
        ws = torch.empty(g.workspace_size(m), dtype=torch.uint8, device="cuda")
        y_ref = g.run(w, x, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ref), f"call {call}: differs from qgemv_run"
        xq, dx, _ = quantize_q8(x_np)
        rows = np.unique(np.linspace(0, n - 1, min(n, 500)).astype(np.int64))
        ref = og.gemv_rows(fmt, synth.weights(fmt, n, k, seed=900), n, k, rows, xq, dx)
        assert normwise(host(y_na)[:, rows], ref) <= TOL


def test_noalloc_second_plan_smaller_input():
    # Two plans in a row on the same scratch: a large call, then a smaller
    # plan whose workspace is a prefix of what the first left behind.
    big, small = ("q8_0", 3000, 8192, 16), ("iq4_nl", 500, 1024, 1)
    outs = []
    for fmt, n, k, m in (big, small):
        cb = synth.codebook(77) if fmt == "iq4_nl" else None
        g = qg.GEMV(fmt, n, k, max_m=m, codebook=cb)
        w = dev(synth.weights(fmt, n, k, seed=910))
        x = dev(synth.activations(911, m, k))
        y_na = g.run_noalloc(w, x)
        y_ref = g.run(w, x, ws=torch.empty(g.workspace_size(m), dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        outs.append(torch.equal(y_na, y_ref))
    assert outs == [True, True]


def test_noalloc_rejects_oversized_workspace():
    g = qg.GEMV("q8_0", 64, 65536, max_m=32)
    assert g.workspace_size(32) > 4 << 20
    w = torch.zeros(g.weight_bytes(0), dtype=torch.uint8, device="cuda")
    x = torch.zeros((32, 65536), dtype=torch.float32, device="cuda")
    with pytest.raises(qg.QgemvError) as ei:
        g.run_noalloc(w, x)
    assert ei.value.status == -5 and "scratch" in str(ei.value)
    # one token of the same plan fits
    y = g.run_noalloc(w, x[:1])
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0
