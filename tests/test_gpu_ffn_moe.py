"""GPU parity of the fused FFN sublayer and the MoE layer, checked stage by
stage against the oracle.

Floating-point noise between the device (fp32) and the oracle (fp64) can
flip a re-quantized code or a top-k choice at a near-tie, so later stages are
checked conditioned on the device's own intermediates (read from the
documented workspace layout), where the oracle takes the same integer
decision in the same precision. The fully independent chain's error is
printed for information.
"""
import numpy as np
import pytest

import synth
from oracle import ffn as offn
from oracle import gemv as og
from oracle import moe as omoe
from oracle.quant import quantize_q8
from tests.gpu_util import TOL, canary_ok, dev, guarded, host, normwise, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import block_quant_gemv_amd as qg  # noqa: E402


def _ws_arrays(plan, ws, m, spec):
    out = {}
    for name, (dtype, count) in spec.items():
        out[name] = host(plan.ws_view(ws, m, name, dtype, count))
    return out


@pytest.mark.parametrize("hidden,inter,m,fgu,fdn", [(4096, 12288, 1, "q4_k", "q6_k"),
                                                    (4096, 256, 1, "q5_k", "q6_k"),
                                                    (6144, 1024, 1, "q4_k", "q4_0"),
                                                    (8192, 4096, 1, "q5_k", "q8_0"),
                                                    (512, 1024, 3, "q4_k", "q6_k"),
                                                    (256, 512, 16, "q4_k", "q6_k"),
                                                    (1024, 2048, 2, "q5_k", "q5_k")])
def test_ffn_staged(hidden, inter, m, fgu, fdn):
    say(f"ffn hidden={hidden} inter={inter} m={m} {fgu}/{fdn}")
    wgu = synth.weights(fgu, 2 * inter, hidden, seed=11)
    wdn = synth.weights(fdn, hidden, inter, seed=12)
    x = synth.activations(13, m, hidden)
    f = qg.FFN(hidden, inter, fgu, fdn, max_m=m)
    ws = f.workspace(m)
    full, y = guarded(torch, m * hidden, torch.float32)
    f.run(dev(wgu), dev(wdn), dev(x), y=y.view(m, hidden), ws=ws)
    torch.cuda.synchronize()
    assert canary_ok(torch, full, m * hidden)
    y = host(y).reshape(m, hidden)
    S = _ws_arrays(f, ws, m, {
        "xq": (torch.int8, m * hidden), "dx": (torch.float32, m * hidden // 32),
        "sx": (torch.int32, m * hidden // 32), "gu": (torch.float32, m * 2 * inter),
        "h": (torch.float32, m * inter), "hq": (torch.int8, m * inter),
        "hd": (torch.float32, m * inter // 32), "hs": (torch.int32, m * inter // 32)})
    # F1: activation codes bit-exact
    xq, dx, sx = quantize_q8(x)
    assert np.array_equal(S["xq"].reshape(m, hidden), xq)
    assert np.array_equal(S["dx"].reshape(m, -1).view(np.int32), dx.view(np.int32))
    assert np.array_equal(S["sx"].reshape(m, -1), sx)
    # F2: gate|up
    gu_ref = og.gemv_dequant(fgu, wgu, 2 * inter, hidden, xq, dx)
    gu = S["gu"].reshape(m, 2 * inter)
    e2 = normwise(gu, gu_ref)
    assert e2 <= TOL, e2
    # F3: SwiGLU on the device's gate|up, re-quantized in the same precision
    h_ref = offn.swiglu(gu, inter)
    h = S["h"].reshape(m, inter)
    assert normwise(h, h_ref) <= 1e-6
    hq, hd, hs = quantize_q8(h)
    assert np.array_equal(S["hq"].reshape(m, inter), hq)
    assert np.array_equal(S["hd"].reshape(m, -1).view(np.int32), hd.view(np.int32))
    assert np.array_equal(S["hs"].reshape(m, -1), hs)
    # F4 (graded): down on the device's re-quantized h
    y_ref = og.gemv_dequant(fdn, wdn, hidden, inter, hq, hd)
    e4 = normwise(y, y_ref)
    # F5 (information): fully independent chain
    full_ref = offn.ffn_ref(wgu, wdn, x, hidden, inter, fgu, fdn)
    flips = int((full_ref["hq"] != hq).sum())
    say(f"  F2 {e2:.2e}  F4 {e4:.2e}  independent {normwise(y, full_ref['y']):.2e} (h code flips {flips})")
    assert e4 <= TOL


def test_ffn_repeated_calls_and_graph_replays():
    # Starting from a workspace of 0xFF bytes (nothing may rely on a cleared
    # workspace), repeated eager calls and graph replays (with eager calls in
    # between) must reproduce each input's result bit for bit, and the last
    # eager result must match the oracle on the device's codes.
    hidden, inter = 4096, 12288
    wgu = dev(synth.weights("q4_k", 2 * inter, hidden, seed=21))
    wdn_np = synth.weights("q6_k", hidden, inter, seed=22)
    wdn = dev(wdn_np)
    f = qg.FFN(hidden, inter)
    ws = f.workspace(1)
    ws.fill_(255)
    xs = [dev(synth.activations(800 + i, 1, hidden)) for i in range(3)]
    eager = [f.run(wgu, wdn, x, ws=ws).clone() for x in xs]
    torch.cuda.synchronize()
    hq = host(f.ws_view(ws, 1, "hq", torch.int8, inter))[None]
    hd = host(f.ws_view(ws, 1, "hd", torch.float32, inter // 32))[None]
    e = normwise(host(eager[2]), og.gemv_dequant("q6_k", wdn_np, hidden, inter, hq, hd))
    say(f"  last eager call vs oracle on the device's codes {e:.2e}")
    assert e <= TOL
    for i in range(3):
        assert torch.equal(f.run(wgu, wdn, xs[i], ws=ws), eager[i]), f"eager repeat {i}"
    x_in = xs[0].clone()
    y_out = torch.empty((1, hidden), dtype=torch.float32, device="cuda")
    f.run(wgu, wdn, x_in, y=y_out, ws=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f.run(wgu, wdn, x_in, y=y_out, ws=ws)
    for rep in range(3):
        for i in (2, 0, 1):
            x_in.copy_(xs[i])
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_out, eager[i]), f"replay {rep} input {i}"
            other = f.run(wgu, wdn, xs[(i + 1) % 3], ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(other, eager[(i + 1) % 3])


def _moe_inputs(E, H, I, seed, fmt="q4_0"):
    gu_all, dn_all = synth.moe_experts(seed, E, H, I, fmt)
    gu_sh, dn_sh = synth.moe_experts(seed + 1, 1, H, I, fmt)
    wr = synth.router_weights(seed + 2, E, H)
    return wr, gu_all, dn_all, gu_sh, dn_sh


# Shapes: the decode workload at 1, 4, 8 and 16 tokens (two-launch expert
# stage); small shapes (six launches); other expert formats (Q4_K, IQ4_NL and
# Q5_K through the two-launch stage, Q8_0 through the six launches, also at
# 16 tokens: its 2176-byte rows do not fit the stage's LDS).
@pytest.mark.parametrize("E,H,I,K,m,fmt", [(256, 2048, 512, 8, 1, "q4_0"), (256, 2048, 512, 8, 4, "q4_0"),
                                            (256, 2048, 512, 8, 8, "q4_0"),
                                            (256, 2048, 512, 8, 16, "q4_0"), (32, 2048, 512, 8, 16, "q8_0"),
                                            (16, 256, 64, 4, 5, "q4_0"), (8, 512, 128, 8, 2, "q4_0"),
                                            (32, 2048, 512, 8, 3, "q8_0"), (32, 2048, 1024, 6, 2, "q4_k"),
                                            (16, 2048, 512, 4, 2, "iq4_nl"), (16, 2048, 512, 8, 3, "q5_k")])
def test_moe_staged(E, H, I, K, m, fmt):
    say(f"moe E={E} H={H} I={I} top{K} m={m} {fmt}")
    wr, gu_all, dn_all, gu_sh, dn_sh = _moe_inputs(E, H, I, seed=31, fmt=fmt)
    x = synth.activations(33, m, H)
    cb = synth.codebook(77) if fmt == "iq4_nl" else None
    mo = qg.MoE(H, I, E, K, fmt, max_m=m, codebook=cb)
    ws = mo.workspace(m)
    full, y = guarded(torch, m * H, torch.float32)
    mo.run(dev(wr), dev(gu_all), dev(dn_all), dev(gu_sh), dev(dn_sh), dev(x), y=y.view(m, H), ws=ws)
    torch.cuda.synchronize()
    assert canary_ok(torch, full, m * H)
    y = host(y).reshape(m, H)
    S1 = K + 1
    S = _ws_arrays(mo, ws, m, {
        "logits": (torch.float32, m * E), "ids": (torch.int32, m * K), "wts": (torch.float32, m * K),
        "xq": (torch.int8, m * H), "dx": (torch.float32, m * H // 32),
        "gu": (torch.float32, m * S1 * 2 * I), "h": (torch.float32, m * S1 * I),
        "hq": (torch.int8, m * S1 * I), "hd": (torch.float32, m * S1 * I // 32)})
    # M1: router logits
    lg = S["logits"].reshape(m, E)
    lg_ref = omoe.router_logits(wr, x)
    assert normwise(lg, lg_ref) <= TOL
    # M2: ids are the top-k of the device logits (ties to the lower index) and
    # equal the oracle's unless the oracle's own ranking has a near-tie.
    ids = S["ids"].reshape(m, K).astype(np.int64)
    assert np.array_equal(ids, omoe.topk(lg.astype(np.float64), K))
    ids_ref = omoe.topk(lg_ref, K)
    for t in range(m):
        if not np.array_equal(ids[t], ids_ref[t]):
            srt = np.sort(lg_ref[t])[::-1]
            assert np.min(np.abs(np.diff(srt[:K + 1]))) < 1e-5, f"token {t}: top-k differs without a near-tie"
    # M3: weights = softmax over the device's selected logits
    wts = S["wts"].reshape(m, K)
    assert normwise(wts, omoe.topk_weights(lg.astype(np.float64), ids)) <= TOL
    # activations
    xq, dx, _ = quantize_q8(x)
    assert np.array_equal(S["xq"].reshape(m, H), xq)
    rb_gu, rb_dn = synth.row_bytes(fmt, H), synth.row_bytes(fmt, I)
    sz_gu, sz_dn = 2 * I * rb_gu, H * rb_dn
    gu_ws = S["gu"].reshape(m, S1, 2 * I)
    h_ws = S["h"].reshape(m, S1, I)
    hq_ws = S["hq"].reshape(m, S1, I)
    hd_ws = S["hd"].reshape(m, S1, I // 32)
    y_cond = np.zeros((m, H))
    for t in range(m):
        outs = []
        for k in range(S1):
            if k < K:
                e = int(ids[t, k])
                wg, wd_ = gu_all[e * sz_gu:(e + 1) * sz_gu], dn_all[e * sz_dn:(e + 1) * sz_dn]
            else:
                wg, wd_ = gu_sh, dn_sh
            # M4: gate|up, SwiGLU + requant (same precision), down on device codes
            g_ref = og.gemv_dequant(fmt, wg, 2 * I, H, xq[t:t + 1], dx[t:t + 1], cb)
            assert normwise(gu_ws[t, k], g_ref[0]) <= TOL
            hq, hd, _ = quantize_q8(h_ws[t, k][None])
            assert np.array_equal(hq_ws[t, k], hq[0])
            assert np.array_equal(hd_ws[t, k].view(np.int32), hd[0].view(np.int32))
            outs.append(og.gemv_dequant(fmt, wd_, H, I, hq, hd, cb)[0])
        y_cond[t] = omoe.combine(outs[:K], wts[t].astype(np.float64), outs[K])
    # M5 (graded)
    e5 = normwise(y, y_cond)
    # M6 (information): fully independent chain
    if fmt == "q4_0":
        ref = omoe.moe_ref(wr, gu_all, dn_all, gu_sh, dn_sh, x, H, I, K)
        say(f"  M5 {e5:.2e}  independent {normwise(y, ref['y']):.2e}")
    assert e5 <= TOL


def test_graph_replays_match_eager():
    # The library only enqueues kernels (no memsets, no host sync), so its
    # calls can be captured in a HIP graph. Replay several times with eager
    # work and synchronisations in between; every replay must equal eager.
    H, I, E, K, m = 512, 128, 16, 4, 3
    wr, gu_all, dn_all, gu_sh, dn_sh = _moe_inputs(E, H, I, seed=41)
    x = dev(synth.activations(42, m, H))
    mo = qg.MoE(H, I, E, K, "q4_0", max_m=m)
    args = [dev(a) for a in (wr, gu_all, dn_all, gu_sh, dn_sh)]
    g = qg.GEMV("q4_k", 512, 2048)
    wg = dev(synth.weights("q4_k", 512, 2048, seed=43))
    xg = dev(synth.activations(44, 1, 2048))
    y_moe = torch.empty((m, H), dtype=torch.float32, device="cuda")
    y_gemv = torch.empty((1, 512), dtype=torch.float32, device="cuda")
    mo.run(*args, x, y=y_moe)
    g.run(wg, xg, y=y_gemv)
    torch.cuda.synchronize()
    ref_moe, ref_gemv = y_moe.clone(), y_gemv.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mo.run(*args, x, y=y_moe)
        g.run(wg, xg, y=y_gemv)
    for rep in range(4):
        y_moe.zero_()
        y_gemv.zero_()
        g.run(wg, dev(synth.activations(45 + rep, 1, 2048)))   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_moe, ref_moe), f"replay {rep}: MoE differs"
        assert torch.equal(y_gemv, ref_gemv), f"replay {rep}: GEMV differs"
