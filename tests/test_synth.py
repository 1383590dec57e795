"""The seeded generators produce the stated distributions (decoded with the
oracle), and the stated model shapes match the cited page facts."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import formats


def test_sizes_agree_with_oracle():
    for fmt in synth.FORMATS:
        for k in (256, 512, 4096):
            assert synth.row_bytes(fmt, k) == formats.row_bytes(fmt, k)
        raw = synth.weights(fmt, 7, 512, seed=0)
        assert raw.size == synth.padded_bytes(fmt, 7, 512) and raw.size % 16 == 0


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_weight_distributions(fmt):
    n, k = 64, 2048
    raw = synth.weights(fmt, n, k, seed=12)
    f = formats.decode(fmt, raw, n, k)
    lo, hi = np.float16(1e-3), np.float16(1e-2)
    assert f["d"].min() >= float(lo) and f["d"].max() <= float(hi)
    q = f["q"]
    if fmt in ("q4_0", "iq4_nl", "q4_k", "iq4_xs"):
        assert q.min() == 0 and q.max() == 15
    elif fmt == "q5_k":
        assert q.min() == 0 and q.max() == 31
    elif fmt == "q8_0":
        assert q.min() == -127 and q.max() == 127
    else:
        assert q.min() == 0 and q.max() == 63
        assert f["sc"].min() == -64 and f["sc"].max() == 63
    if fmt == "iq4_xs":
        assert f["ls"].min() == 0 and f["ls"].max() == 63
    if fmt in ("q4_k", "q5_k"):
        assert f["dmin"].min() >= float(lo) and f["dmin"].max() <= float(hi)
        assert f["sc"].min() == 0 and f["sc"].max() == 63
        assert f["m"].min() == 0 and f["m"].max() == 63
    # roughly uniform codes
    counts = np.bincount((q - q.min()).reshape(-1))
    assert counts.min() > 0.8 * counts.mean()


def test_codebook():
    for seed in range(5):
        cb = synth.codebook(seed)
        assert cb.dtype == np.int8 and cb.size == 16
        assert cb[0] == -127 and cb[-1] == 113
        assert np.all(np.diff(cb.astype(int)) > 0)


def test_seeded_and_deterministic():
    a = synth.weights("q4_k", 5, 256, seed=3)
    b = synth.weights("q4_k", 5, 256, seed=3)
    c = synth.weights("q4_k", 5, 256, seed=4)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    x = synth.activations(1, 2, 64)
    assert x.dtype == np.float32 and np.array_equal(x, synth.activations(1, 2, 64))


def test_moe_shapes_follow_page_facts():
    facts = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))
    s = facts["moe_shapes"]
    assert (s["hidden"], s["n_experts"], s["routed_active"], s["shared_active"],
            s["expert_intermediate"]) == (2048, 256, 8, 1, 512)
    gu, dn = synth.moe_experts(0, 4, 256, 64)
    assert gu.size >= 4 * 2 * 64 * synth.row_bytes("q4_0", 256)
    assert dn.size >= 4 * 256 * synth.row_bytes("q4_0", 64)
