"""GPU parity of the activation quantizer and the five GEMV kernels against
the oracle: quantized activations bit-exact, per-block int32 dot products
bit-exact, fp32 outputs within 2e-5 normwise relative error."""
import numpy as np
import pytest

import synth
from oracle import gemv as og
from oracle.quant import quantize_q8
from tests.gpu_util import TOL, canary_ok, dev, guarded, host, normwise, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import block_quant_gemv_amd as qg  # noqa: E402

CB_SEED = 77
CB_FORMATS = ("iq4_nl", "iq4_xs")


def _codebook():
    return synth.codebook(CB_SEED)


# ------------------------------------------------------------ quantizer --

@pytest.mark.parametrize("seed,m,k", [(0, 1, 32), (1, 1, 2048), (2, 3, 4096), (3, 2, 12288), (4, 16, 2048)])
def test_quantizer_bit_exact(seed, m, k):
    say(f"quantizer seed={seed} m={m} k={k}")
    x = synth.activations(seed, m, k)
    x[0, :32] = np.float32(0)                       # zero block
    if k >= 64:
        x[0, 32:64] = np.float32(0.5) * np.arange(32, dtype=np.float32) - np.float32(7.5)  # ties
        x[0, 63] = np.float32(127.0)
    xq, dx, sx = qg.debug_quantize(dev(x))
    torch.cuda.synchronize()
    rq, rd, rs = quantize_q8(x)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(dx).view(np.int32), rd.view(np.int32))
    assert np.array_equal(host(sx), rs)


def _near_tie_blocks():
    """Blocks whose elements sit at, and a few ulps around, the fp32 values
    closest to (k + 1/2) * d for many k and several scales d: the cases where
    the code depends on the correctly rounded quotient."""
    rows = []
    for a in (np.float32(127.0), np.float32(100.0), np.float32(3.1), np.float32(0.017), np.float32(5e-30)):
        d = np.float32(a) / np.float32(127)
        ks = np.arange(-126, 126)
        base = ((ks + 0.5) * np.float64(d)).astype(np.float32)
        cands = [base]
        for step in (1, 2, 3):
            up = base.copy()
            dn = base.copy()
            for _ in range(step):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
            cands += [up, dn]
        vals = np.concatenate(cands)
        vals = vals[np.abs(vals) < a]
        nblk = -(-vals.size // 31)
        blk = np.zeros((nblk, 32), np.float32)
        flat = np.zeros(nblk * 31, np.float32)
        flat[: vals.size] = vals
        blk[:, 1:] = flat.reshape(nblk, 31)
        blk[:, 0] = a
        rows.append(blk.reshape(-1))
    x = np.concatenate(rows)
    pad = (-x.size) % 32
    return np.concatenate([x, np.zeros(pad, np.float32)])[None, :]


def test_quantizer_near_ties_bit_exact():
    x = _near_tie_blocks()
    say(f"quantizer near ties: {x.size} elements")
    xq, dx, sx = qg.debug_quantize(dev(x))
    torch.cuda.synchronize()
    rq, rd, rs = quantize_q8(x)
    assert np.array_equal(host(dx).view(np.int32), rd.view(np.int32))
    bad = np.argwhere(host(xq) != rq)
    assert bad.size == 0, f"{len(bad)} codes differ, e.g. {bad[:5].tolist()}"
    assert np.array_equal(host(sx), rs)


@pytest.mark.parametrize("fmt,k,n", [("q8_0", 2048, 64), ("q6_k", 2048, 64), ("q8_0", 4096, 4096),
                                     ("q4_k", 4096, 4096), ("q6_k", 12288, 1024)])
def test_fused_quantize_writes_workspace_codes(fmt, k, n):
    # qgemv_run quantizes x (inside the GEMV kernel for short rows, in a
    # launch of its own for long ones); the codes it leaves in the workspace
    # must equal the standalone rule bit for bit.
    ties = _near_tie_blocks()
    x = np.concatenate([ties, synth.activations(3, 1, max(0, k - ties.shape[1]))], axis=1)[:, :k]
    w = synth.weights(fmt, n, k, seed=2)
    g = qg.GEMV(fmt, n, k)
    ws = g.workspace(1)
    g.run(dev(w), dev(x), ws=ws)
    torch.cuda.synchronize()
    rq, rd, rs = quantize_q8(x)
    assert np.array_equal(host(g.ws_view(ws, 1, "xq", torch.int8, k)), rq[0])
    assert np.array_equal(host(g.ws_view(ws, 1, "dx", torch.float32, k // 32)).view(np.int32), rd[0].view(np.int32))
    assert np.array_equal(host(g.ws_view(ws, 1, "sx", torch.int32, k // 32)), rs[0])


# ----------------------------------------------------------------- GEMV --

SMALL = [
    # fmt, n, k, m
    ("q4_0", 2048, 2048, 1),      # the Q4_0 decode GEMV, full size
    ("q4_0", 257, 288, 1),        # ragged: 9 blocks per row, odd rows
    ("q4_0", 20, 32, 3),
    ("q4_0", 1, 512, 2),
    ("q8_0", 4096, 4096, 1),      # dense-layer shape
    ("q8_0", 257, 288, 2),
    ("q8_0", 33, 16384, 1),       # long rows: K-segmented steps
    ("q4_k", 4096, 4096, 1),
    ("q4_k", 20, 256, 3),
    ("q4_k", 257, 768, 1),
    ("q4_k", 9, 12288, 16),
    ("q4_k", 333, 2048, 1),       # register-direct single-token kernel: K = 2048 ... 8192
    ("q4_k", 3, 6144, 1),
    ("q4_k", 4097, 8192, 1),
    ("q4_k", 8195, 4096, 1),      # four-row groups with a ragged last group
    ("q6_k", 4096, 12288, 1),     # FFN down shape
    ("q6_k", 20, 256, 1),
    ("q6_k", 257, 512, 4),
    ("q6_k", 7, 16384, 2),        # long rows
    ("iq4_nl", 4096, 4096, 1),
    ("iq4_nl", 257, 288, 1),
    ("iq4_nl", 20, 32, 8),
    # K > 2048 with several tokens, token chunks and tiny grids
    ("q8_0", 2048, 4096, 4),
    ("iq4_nl", 1500, 6144, 3),
    ("q6_k", 1024, 12288, 8),
    ("q8_0", 1000, 4096, 16),
    ("q4_0", 700, 8192, 2),
    ("q8_0", 8, 4096, 1),
    # Q5_K and IQ4_XS: the formats the pages' single-matrix bandwidth figures
    # are quoted on (full-size shape, ragged rows, several tokens, long rows)
    ("q5_k", 4096, 4096, 1),
    ("q5_k", 257, 768, 3),
    ("q5_k", 20, 256, 16),
    ("q5_k", 33, 16384, 2),
    ("q5_k", 333, 2048, 1),       # register-direct kernel: K = 2048 ... 8192,
    ("q5_k", 8195, 4096, 1),      # four-row groups with a ragged last group
    ("q5_k", 4097, 8192, 1),
    ("iq4_xs", 4096, 4096, 1),
    ("iq4_xs", 257, 768, 2),     # 3 super-blocks per row: 8-byte aligned rows
    ("iq4_xs", 20, 256, 8),
    ("iq4_xs", 9, 16640, 1),     # 65 super-blocks per row, K-segmented
]


def _run_case(fmt, n, k, m, seed):
    cb = _codebook() if fmt in CB_FORMATS else None
    w = synth.weights(fmt, n, k, seed=seed)
    x = synth.activations(seed + 1, m, k)
    g = qg.GEMV(fmt, n, k, max_m=max(m, 1), codebook=cb)
    wd = dev(w)
    full, y = guarded(torch, m * n, torch.float32)
    g.run(wd, dev(x), y.view(m, n))
    xq, dx, sx = quantize_q8(x)
    dots = g.block_dots(wd, dev(xq))
    torch.cuda.synchronize()
    return g, w, x, xq, dx, sx, host(y).reshape(m, n), host(dots), canary_ok(torch, full, m * n), cb


@pytest.mark.parametrize("fmt,n,k,m", SMALL)
def test_gemv_parity(fmt, n, k, m):
    say(f"gemv {fmt} n={n} k={k} m={m}")
    g, w, x, xq, dx, sx, y, dots, canary, cb = _run_case(fmt, n, k, m, seed=n + k + m)
    assert canary, "output guard band overwritten"
    ref_dots = og.block_dots(fmt, w, n, k, xq, cb)
    assert dots.shape == ref_dots.shape
    bad = np.argwhere(dots != ref_dots)
    assert bad.size == 0, f"{len(bad)} block dots differ, first {bad[:3].tolist()}"
    ref = og.gemv_dequant(fmt, w, n, k, xq, dx, cb)
    e = normwise(y, ref)
    say(f"  normwise error {e:.3e}")
    assert e <= TOL


@pytest.mark.parametrize("fmt,n,k", [("q8_0", 12288, 4096), ("q8_0", 24576, 4096),
                                     ("q4_k", 12288, 4096), ("q4_k", 24576, 4096),
                                     ("iq4_nl", 248320, 4096), ("q5_k", 12288, 4096),
                                     ("iq4_xs", 12288, 4096)])
def test_gemv_full_size_sampled_rows(fmt, n, k):
    say(f"gemv full size {fmt} n={n} k={k}")
    cb = _codebook() if fmt in CB_FORMATS else None
    w = synth.weights(fmt, n, k, seed=101)
    x = synth.activations(102, 1, k)
    g = qg.GEMV(fmt, n, k, codebook=cb)
    wd = dev(w)
    y = host(g.run(wd, dev(x)))
    torch.cuda.synchronize()
    xq, dx, _ = quantize_q8(x)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, n // 2, n - 2, n - 1], rng.integers(0, n, 2000)]))
    ref = og.gemv_rows(fmt, w, n, k, rows, xq, dx, cb)
    e = normwise(y[:, rows], ref)
    say(f"  sampled normwise error {e:.3e} over {rows.size} rows")
    assert e <= TOL
    # per-row relative error on the sample
    assert np.all(np.abs(y[0, rows] - ref[0]) <= 1e-4 * (np.abs(ref[0]) + np.abs(ref[0]).mean()))


def test_repeated_calls_shared_workspace():
    # Plans with different kernels and grids take turns on one workspace;
    # every call must see its own codes.
    k = 4096
    cases = [("q8_0", 4096), ("q4_k", 8195), ("iq4_nl", 300), ("q8_0", 8)]
    cb = _codebook()
    plans, weights = [], []
    for i, (fmt, n) in enumerate(cases):
        plans.append(qg.GEMV(fmt, n, k, codebook=cb if fmt == "iq4_nl" else None))
        weights.append(synth.weights(fmt, n, k, seed=40 + i))
    wsz = max(p.workspace_size(1) for p in plans)
    assert all(p.workspace_size(1) == wsz for p in plans)
    ws = torch.zeros(wsz, dtype=torch.uint8, device="cuda")
    wds = [dev(w) for w in weights]
    for it in range(2):
        for i, ((fmt, n), g) in enumerate(zip(cases, plans)):
            say(f"shared workspace round {it} {fmt} n={n}")
            x = synth.activations(600 + 10 * it + i, 1, k)
            y = host(g.run(wds[i], dev(x), ws=ws))
            torch.cuda.synchronize()
            xq, dx, sx = quantize_q8(x)
            assert np.array_equal(host(g.ws_view(ws, 1, "xq", torch.int8, k)), xq[0])
            assert np.array_equal(host(g.ws_view(ws, 1, "sx", torch.int32, k // 32)), sx[0])
            rows = np.unique(np.linspace(0, n - 1, min(n, 600)).astype(np.int64))
            ref = og.gemv_rows(fmt, weights[i], n, k, rows, xq, dx, cb if fmt == "iq4_nl" else None)
            assert normwise(y[:, rows], ref) <= TOL


def test_graph_replays_match_eager():
    # Captured once, replayed with new inputs, with eager calls on the same
    # workspace in between: every replay matches the eager result bit for bit.
    fmt, n, k = "q8_0", 4096, 4096
    w = dev(synth.weights(fmt, n, k, seed=50))
    g = qg.GEMV(fmt, n, k)
    ws = g.workspace(1)
    xs = [dev(synth.activations(700 + i, 1, k)) for i in range(3)]
    eager = [g.run(w, x, ws=ws).clone() for x in xs]
    x_in = xs[0].clone()
    y_out = torch.empty((1, n), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    g.run(w, x_in, y=y_out, ws=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        g.run(w, x_in, y=y_out, ws=ws)
    for rep in range(3):
        for i in (2, 0, 1):
            x_in.copy_(xs[i])
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_out, eager[i]), f"replay {rep} input {i}"
            other = g.run(w, xs[(i + 1) % 3], ws=ws)  # eager call between replays
            torch.cuda.synchronize()
            assert torch.equal(other, eager[(i + 1) % 3])


def test_gemv_deterministic_and_workspace_guard():
    fmt, n, k = "q4_k", 4096, 4096
    w = dev(synth.weights(fmt, n, k, seed=3))
    x = dev(synth.activations(4, 2, k))
    g = qg.GEMV(fmt, n, k, max_m=2)
    wsz = g.workspace_size(2)
    full, ws = guarded(torch, wsz, torch.uint8, pad=4096)
    ws.zero_()  # a workspace starts zero-filled
    y1 = g.run(w, x, ws=ws).clone()
    y2 = g.run(w, x, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert canary_ok(torch, full, wsz, pad=4096)


def test_gemv_many_tokens_chunked():
    # m = 32 with a format that has no MFMA path runs the VALU kernel in chunks.
    fmt, n, k, m = "q8_0", 300, 512, 32
    w = synth.weights(fmt, n, k, seed=8)
    x = synth.activations(9, m, k)
    g = qg.GEMV(fmt, n, k, max_m=m)
    y = host(g.run(dev(w), dev(x)))
    xq, dx, _ = quantize_q8(x)
    assert normwise(y, og.gemv_dequant(fmt, w, n, k, xq, dx)) <= TOL


def test_single_hip_runtime_loaded():
    maps = open("/proc/self/maps").read()
    libs = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(libs) == 1, libs
    assert any("libqgemv.so" in ln for ln in maps.splitlines())


# ------------------------------------------------------- M = 32, int8 MFMA --

@pytest.mark.parametrize("fmt,n,k,m", [("q4_k", 12288, 4096, 32),    # batched shape, Q4_K
                                       ("q6_k", 4096, 12288, 32),    # batched shape, Q6_K
                                       ("q4_k", 100, 512, 17),       # ragged rows, odd tokens
                                       ("q6_k", 33, 1280, 20),       # K not a multiple of the split
                                       ("q4_k", 64, 256, 32)])
def test_mfma_batched_parity(fmt, n, k, m):
    say(f"mfma {fmt} n={n} k={k} m={m}")
    w = synth.weights(fmt, n, k, seed=n + m)
    x = synth.activations(k + m, m, k)
    g = qg.GEMV(fmt, n, k, max_m=32)
    wd = dev(w)
    full, y = guarded(torch, m * n, torch.float32)
    g.run(wd, dev(x), y.view(m, n))
    xq, dx, sx = quantize_q8(x)
    dots = host(g.block_dots(wd, dev(xq)))
    torch.cuda.synchronize()
    assert canary_ok(torch, full, m * n)
    ref_dots = og.block_dots(fmt, w, n, k, xq)
    bad = np.argwhere(dots != ref_dots)
    assert bad.size == 0, f"{len(bad)} MFMA block dots differ, first {bad[:3].tolist()}"
    ref = og.gemv_dequant(fmt, w, n, k, xq, dx)
    e = normwise(host(y).reshape(m, n), ref)
    say(f"  normwise error {e:.3e}")
    assert e <= TOL


def _random_cases(count, seed):
    # Seeded random shapes within the library's limits: every format, row
    # counts that are not multiples of any tile, K from one block (or
    # super-block) to 8192, 1..32 tokens (MFMA path from 9 tokens for Q4_K
    # and Q6_K, token chunks above 16 for the others).
    rng = np.random.default_rng(seed)
    fmts = ["q4_0", "q8_0", "q4_k", "q6_k", "iq4_nl", "q5_k", "iq4_xs"]
    out = []
    for i in range(count):
        fmt = fmts[i % len(fmts)]
        be = 256 if fmt in ("q4_k", "q6_k", "q5_k", "iq4_xs") else 32
        k = be * int(rng.integers(1, 8192 // be + 1))
        n = int(rng.integers(1, 3000))
        m = int(rng.choice([1, 1, 2, 3, 5, 8, 13, 17, 32]))
        n = max(1, min(n, int(1.5e8 // (m * k))))  # keeps the oracle's integer dots to seconds
        out.append((fmt, n, k, m))
    return out


@pytest.mark.parametrize("fmt,n,k,m", _random_cases(28, 2026))
def test_gemv_random_shapes(fmt, n, k, m):
    say(f"random gemv {fmt} n={n} k={k} m={m}")
    g, w, x, xq, dx, sx, y, dots, canary, cb = _run_case(fmt, n, k, m, seed=n * 7 + k + m)
    assert canary, "output guard band overwritten"
    assert np.array_equal(dots, og.block_dots(fmt, w, n, k, xq, cb))
    assert normwise(y, og.gemv_dequant(fmt, w, n, k, xq, dx, cb)) <= TOL
