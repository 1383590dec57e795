"""GPU parity of the MoE layer with 16-bit activations (qmoe_run_s16), stage
by stage against the oracle, conditioned on the device's own intermediates
where a re-quantized code or a top-k choice could sit at a near-tie; and its
accuracy against the MoE layer with unquantized activations, next to the
int8 layer's."""
import numpy as np
import pytest

import synth
from oracle import gemv as og
from oracle import moe as omoe
from oracle.ffn import swiglu
from oracle.quant import quantize_s16
from tests.gpu_util import TOL, canary_ok, dev, guarded, host, normwise, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import block_quant_gemv_amd as qg  # noqa: E402


def _inputs(E, H, I, seed):
    gu_all, dn_all = synth.moe_experts(seed, E, H, I)
    gu_sh, dn_sh = synth.moe_experts(seed + 1, 1, H, I)
    wr = synth.router_weights(seed + 2, E, H)
    return wr, gu_all, dn_all, gu_sh, dn_sh


# Shapes: the decode workload at 1, 4, 12 and 16 tokens (the two-launch
# expert stage up to 13 tokens at hidden 2048, where its LDS holds the staged
# 16-bit codes; six launches at 16), intermediate 1024 through the two-launch
# stage, and small shapes through the six launches.
@pytest.mark.parametrize("E,H,I,K,m", [(256, 2048, 512, 8, 1), (256, 2048, 512, 8, 4), (256, 2048, 512, 8, 12),
                                        (256, 2048, 512, 8, 16), (64, 2048, 1024, 8, 3),
                                        (16, 1024, 512, 4, 5), (8, 512, 1024, 8, 2)])
def test_moe_s16_staged(E, H, I, K, m):
    say(f"moe s16 E={E} H={H} I={I} top{K} m={m}")
    wr, gu_all, dn_all, gu_sh, dn_sh = _inputs(E, H, I, seed=41)
    x = synth.activations(43, m, H)
    mo = qg.MoE(H, I, E, K, "q4_0", max_m=m)
    ws = mo.workspace(m)
    full, y = guarded(torch, m * H, torch.float32)
    mo.run(dev(wr), dev(gu_all), dev(dn_all), dev(gu_sh), dev(dn_sh), dev(x), y=y.view(m, H), ws=ws, s16=True)
    torch.cuda.synchronize()
    assert canary_ok(torch, full, m * H)
    y = host(y).reshape(m, H)
    S1 = K + 1

    def view(name, dtype, count):
        return host(mo.ws_view(ws, m, name, dtype, count))

    lg = view("logits", torch.float32, m * E).reshape(m, E)
    assert normwise(lg, omoe.router_logits(wr, x)) <= TOL
    ids = view("ids", torch.int32, m * K).reshape(m, K).astype(np.int64)
    assert np.array_equal(ids, omoe.topk(lg.astype(np.float64), K))
    wts = view("wts", torch.float32, m * K).reshape(m, K)
    assert normwise(wts, omoe.topk_weights(lg.astype(np.float64), ids)) <= TOL
    # 16-bit codes of x, bit-exact
    xq, dx, sx = quantize_s16(x)
    assert np.array_equal(view("xq16", torch.int16, m * H).reshape(m, H), xq)
    assert np.array_equal(view("dx", torch.float32, m * H // 32).reshape(m, -1).view(np.int32), dx.view(np.int32))
    assert np.array_equal(view("sx", torch.int32, m * H // 32).reshape(m, -1), sx)
    rb_gu, rb_dn = synth.row_bytes("q4_0", H), synth.row_bytes("q4_0", I)
    sz_gu, sz_dn = 2 * I * rb_gu, H * rb_dn
    gu_ws = view("gu", torch.float32, m * S1 * 2 * I).reshape(m, S1, 2 * I)
    h_ws = view("h", torch.float32, m * S1 * I).reshape(m, S1, I)
    hq_ws = view("hq16", torch.int16, m * S1 * I).reshape(m, S1, I)
    hd_ws = view("hd", torch.float32, m * S1 * I // 32).reshape(m, S1, I // 32)
    hs_ws = view("hs", torch.int32, m * S1 * I // 32).reshape(m, S1, I // 32)
    y_cond = np.zeros((m, H))
    for t in range(m):
        outs = []
        for k in range(S1):
            if k < K:
                e = int(ids[t, k])
                wg, wd_ = gu_all[e * sz_gu:(e + 1) * sz_gu], dn_all[e * sz_dn:(e + 1) * sz_dn]
            else:
                wg, wd_ = gu_sh, dn_sh
            g_ref = og.gemv_dequant("q4_0", wg, 2 * I, H, xq[t:t + 1], dx[t:t + 1])
            assert normwise(gu_ws[t, k], g_ref[0]) <= TOL
            assert normwise(h_ws[t, k], swiglu(gu_ws[t, k][None], I)[0]) <= 1e-6
            hq, hd, hs = quantize_s16(h_ws[t, k][None])
            assert np.array_equal(hq_ws[t, k], hq[0])
            assert np.array_equal(hd_ws[t, k].view(np.int32), hd[0].view(np.int32))
            assert np.array_equal(hs_ws[t, k], hs[0])
            outs.append(og.gemv_dequant("q4_0", wd_, H, I, hq, hd)[0])
        y_cond[t] = omoe.combine(outs[:K], wts[t].astype(np.float64), outs[K])
    e5 = normwise(y, y_cond)
    ref = omoe.moe_ref(wr, gu_all, dn_all, gu_sh, dn_sh, x, H, I, K, quant=quantize_s16)
    say(f"  graded {e5:.2e}  independent {normwise(y, ref['y']):.2e}")
    assert e5 <= TOL


def test_moe_s16_accuracy_vs_int8():
    # Against the layer with unquantized activations (codes = x itself, unit
    # scales), the 16-bit layer errs far less than the int8 one.
    E, H, I, K, m = 64, 2048, 512, 8, 4
    wr, gu_all, dn_all, gu_sh, dn_sh = _inputs(E, H, I, seed=45)
    x = synth.activations(46, m, H)
    mo = qg.MoE(H, I, E, K, "q4_0", max_m=m)
    args = [dev(a) for a in (wr, gu_all, dn_all, gu_sh, dn_sh, x)]
    y16 = host(mo.run(*args, s16=True))
    y8 = host(mo.run(*args))
    torch.cuda.synchronize()

    def exact(v):
        v = np.asarray(v, np.float32)
        return v.astype(np.float64), np.ones((v.shape[0], v.shape[1] // 32), np.float64), None

    ref = omoe.moe_ref(wr, gu_all, dn_all, gu_sh, dn_sh, x, H, I, K, quant=exact)
    e16, e8 = normwise(y16, ref["y"]), normwise(y8, ref["y"])
    say(f"  error vs unquantized activations: s16 {e16:.2e}, int8 {e8:.2e}")
    assert e16 * 50 < e8
