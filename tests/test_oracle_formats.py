"""Pins for the oracle's block layouts.

Hand-planted blocks below are written byte by byte from the layout reading
(documented in oracle/formats.py) and their expected values computed by hand,
so a wrong nibble order, bit offset or field position in the decoder fails
here. Round trips and exhaustive sweeps cover the rest of each code range.
"""
import json
import os

import numpy as np
import pytest

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f16_bytes(v):
    return list(np.array([v], "<f2").view(np.uint8))


def test_block_sizes_and_q4_0_bits_per_weight():
    assert formats.BLOCK_BYTES == {"q4_0": 18, "q8_0": 34, "iq4_nl": 18, "q4_k": 144, "q6_k": 210,
                                   "q5_k": 176, "iq4_xs": 136}
    # bits per weight: Q5_K is Q4_K plus one bit per weight; IQ4_XS is 4.25
    assert formats.BLOCK_BYTES["q5_k"] * 8 == formats.BLOCK_BYTES["q4_k"] * 8 + 256
    assert formats.BLOCK_BYTES["iq4_xs"] * 8 / 256 == 4.25
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    bpw = formats.BLOCK_BYTES["q4_0"] * 8 / formats.BLOCK_ELEMS["q4_0"]
    assert bpw == pytest.approx(facts["q4_0_bits_per_weight"]["value"])
    # row bytes at the workload shapes are multiples of 16
    for fmt, k, rb in [("q4_0", 2048, 1152), ("q4_0", 512, 288), ("q8_0", 4096, 4352),
                       ("q4_k", 4096, 2304), ("iq4_nl", 4096, 2304), ("q6_k", 12288, 10080),
                       ("q5_k", 4096, 2816), ("iq4_xs", 4096, 2176)]:
        assert formats.row_bytes(fmt, k) == rb and rb % 16 == 0


def test_q4_0_planted_block():
    blk = _f16_bytes(1.0) + [0x88] * 16
    blk[2 + 0] = 0x21      # element 0 low nibble 1, element 16 high nibble 2
    blk[2 + 15] = 0xF0     # element 15 -> 0, element 31 -> 15
    v = formats.values("q4_0", np.array(blk, np.uint8), 1, 32)[0]
    exp = np.zeros(32)
    exp[0], exp[16], exp[15], exp[31] = 1 - 8, 2 - 8, 0 - 8, 15 - 8
    assert np.array_equal(v, exp)


def test_q8_0_planted_block():
    codes = [0] * 32
    codes[0], codes[31], codes[5] = -127, 127, -128
    blk = _f16_bytes(0.5) + list(np.array(codes, np.int8).view(np.uint8))
    v = formats.values("q8_0", np.array(blk, np.uint8), 1, 32)[0]
    exp = np.zeros(32)
    exp[0], exp[31], exp[5] = -63.5, 63.5, -64.0
    assert np.array_equal(v, exp)


def test_iq4_nl_planted_block():
    cb = np.array([-127, -100, -80, -60, -40, -20, -10, -1, 0, 5, 15, 30, 50, 70, 90, 113], np.int8)
    blk = _f16_bytes(2.0) + [0x00] * 16
    blk[2 + 3] = 0xF7      # element 3 -> idx 7 (-1), element 19 -> idx 15 (113)
    v = formats.values("iq4_nl", np.array(blk, np.uint8), 1, 32, codebook=cb)[0]
    exp = np.full(32, 2.0 * -127)
    exp[3], exp[19] = 2.0 * -1, 2.0 * 113
    assert np.array_equal(v, exp)


def test_q4_k_planted_block():
    blk = [0] * 144
    blk[0:2] = _f16_bytes(1.0)
    blk[2:4] = _f16_bytes(0.5)
    # scales: 96-bit little-endian stream of 6-bit fields
    # field 0 (sc0) = 1     -> bit 0 of byte 4
    # field 1 (sc1) = 63    -> bits 6..11: byte 4 bits 6,7 and byte 5 bits 0..3
    # field 8 (m0)  = 2     -> bits 48..53: byte 10 bit 1
    # field 15 (m7) = 63    -> bits 90..95: byte 15 bits 2..7
    blk[4] = 0x01 | 0xC0
    blk[5] = 0x0F
    blk[10] = 0x02
    blk[15] = 0xFC
    blk[16] = 0x53          # sub-block 0: element 0 -> 3, element 16 -> 5
    blk[16 + 16 + 2] = 0x0A  # sub-block 1: element 32+2 -> 10
    f = formats.decode("q4_k", np.array(blk, np.uint8), 1, 256)
    assert list(f["sc"][0, 0]) == [1, 63, 0, 0, 0, 0, 0, 0]
    assert list(f["m"][0, 0]) == [2, 0, 0, 0, 0, 0, 0, 63]
    v = formats.values("q4_k", np.array(blk, np.uint8), 1, 256)[0]
    exp = np.zeros(256)
    exp[0:32] = -0.5 * 2            # q = 0 -> -dmin*m0
    exp[0] = 1 * 1 * 3 - 1.0
    exp[16] = 1 * 1 * 5 - 1.0
    exp[32:64] = 0.0                # sc1 = 63 but q = 0, m1 = 0
    exp[34] = 63 * 10
    exp[224:256] = -0.5 * 63        # sub-block 7: sc 0, m 63
    assert np.array_equal(v, exp)


def test_q6_k_planted_block():
    blk = [0] * 210
    blk[0:2] = _f16_bytes(1.0)
    sc = [0] * 16
    sc[0], sc[1], sc[15] = -2, 3, -64
    blk[2:18] = list(np.array(sc, np.int8).view(np.uint8))
    ql, qh = 18, 146
    blk[ql + 0] = 0x21      # element 0 low 1, element 16 low 2
    blk[ql + 8] = 0x43      # element 8 low 3, element 24 low 4
    blk[qh + 0] = 0xE4      # bits 0-1: el 0 hi 0; 2-3: el 8 hi 1; 4-5: el 16 hi 2; 6-7: el 24 hi 3
    blk[ql + 127] = 0xF0    # group 7, i = 31 (element 255) low 15
    blk[qh + 63] = 0xC0     # group 7, i = 31 hi 3  -> q = 63
    v = formats.values("q6_k", np.array(blk, np.uint8), 1, 256)[0]
    exp = np.zeros(256)
    for j in range(16):
        exp[16 * j:16 * j + 16] = sc[j] * (0 - 32)
    exp[0] = -2 * (1 - 32)
    exp[8] = -2 * (19 - 32)
    exp[16] = 3 * (34 - 32)
    exp[24] = 3 * (52 - 32)
    exp[255] = -64 * (63 - 32)
    assert np.array_equal(v, exp)


def test_q5_k_planted_block():
    blk = [0] * 176
    blk[0:2] = _f16_bytes(1.0)
    blk[2:4] = _f16_bytes(0.25)
    blk[4] = 0x02           # sc0 = 2
    blk[10] = 0x04          # m0 = 4 (field 8 at bit 48 = byte 10 bit 0)
    # qh: sub-block j's fifth bits in bytes 16 + 4j .. 16 + 4j + 3; element i
    # of the sub-block at byte i % 4, bit i // 4
    blk[16 + 0] = 0x01      # element 0 (byte 0, bit 0)
    blk[16 + 3] = 0x80      # element 31 (byte 3, bit 7)
    blk[16 + 1] = 0x10      # element 17 (byte 1, bit 4)
    blk[48 + 0] = 0x35      # element 0 low 5; element 16 low 3
    blk[48 + 1] = 0x60      # element 1 low 0; element 17 low 6
    blk[48 + 15] = 0xF0     # element 15 low 0; element 31 low 15
    blk[16 + 4 * 7 + 2] = 0x20  # sub-block 7 element 22 (byte 2, bit 5) -> element 246
    v = formats.values("q5_k", np.array(blk, np.uint8), 1, 256)[0]
    exp = np.zeros(256)
    exp[0:32] = -0.25 * 4                 # q = 0: -dmin * m0
    exp[0] = 2 * (5 + 16) - 1.0
    exp[16] = 2 * 3 - 1.0
    exp[17] = 2 * (6 + 16) - 1.0
    exp[31] = 2 * (15 + 16) - 1.0
    exp[246] = 0.0                        # sub-block 7: sc = 0, m = 0
    assert np.array_equal(v, exp)
    f = formats.decode("q5_k", np.array(blk, np.uint8), 1, 256)
    assert f["q"][0, 0, 246] == 16 and f["q"][0, 0, 1] == 0


def test_iq4_xs_planted_block():
    cb = np.array([-127, -100, -80, -60, -40, -20, -10, -1, 0, 5, 15, 30, 50, 70, 90, 113], np.int8)
    blk = [0] * 136
    blk[0:2] = _f16_bytes(0.5)
    # ls_0 = 33 (low 1, high 2), ls_1 = 0, ls_7 = 63 (low 15, high 3)
    blk[4] = 0x01                               # scales_l[0]: ls_0 low 1, ls_1 low 0
    blk[7] = 0xF0                               # scales_l[3]: ls_6 low 0, ls_7 low 15
    sh = (2 << 0) | (3 << 14)
    blk[2], blk[3] = sh & 0xFF, sh >> 8
    blk[8 + 0] = 0xF9                           # element 0 -> idx 9 (5); element 16 -> idx 15 (113)
    blk[8 + 16 * 7 + 3] = 0x07                  # sub-block 7, element 3 -> idx 7 (-1); element 19 -> idx 0
    f = formats.decode("iq4_xs", np.array(blk, np.uint8), 1, 256, codebook=cb)
    assert list(f["ls"][0, 0]) == [33, 0, 0, 0, 0, 0, 0, 63]
    v = formats.values("iq4_xs", np.array(blk, np.uint8), 1, 256, codebook=cb)[0]
    exp = np.zeros(256)
    exp[0:32] = 0.5 * 1 * -127               # ls 33 -> scale 1, idx 0
    exp[0] = 0.5 * 5
    exp[16] = 0.5 * 113
    exp[32:64] = 0.5 * -32 * -127            # ls_1 = 0 -> scale -32
    for j in range(2, 7):
        exp[32 * j:32 * j + 32] = 0.5 * -32 * -127   # ls 0 elsewhere
    exp[224:256] = 0.5 * 31 * -127            # ls_7 = 63 -> 31
    exp[224 + 3] = 0.5 * 31 * -1
    assert np.array_equal(v, exp)


def test_q5_k_with_zero_fifth_bits_is_q4_k():
    # the same fields through the two decoders (different code offsets)
    n, k = 4, 512
    rng = np.random.default_rng(17)
    nb = k // 256
    f = {"d": rng.uniform(1e-3, 1e-2, (n, nb)).astype(np.float16).astype(np.float64),
         "dmin": rng.uniform(1e-3, 1e-2, (n, nb)).astype(np.float16).astype(np.float64),
         "sc": rng.integers(0, 64, (n, nb, 8)), "m": rng.integers(0, 64, (n, nb, 8)),
         "q": rng.integers(0, 16, (n, nb, 256))}
    v4 = formats.values("q4_k", formats.encode("q4_k", f), n, k)
    v5 = formats.values("q5_k", formats.encode("q5_k", f), n, k)
    assert np.array_equal(v4, v5)
    # every fifth bit set adds 16 * d * sc_j to every element
    raw5 = formats.encode("q5_k", dict(f, q=f["q"] + 16))
    v5b = formats.values("q5_k", raw5, n, k).reshape(n, nb, 8, 32)
    add = (16 * f["d"][..., None] * f["sc"])[..., None]
    assert np.allclose(v5b - v4.reshape(n, nb, 8, 32), add, rtol=0, atol=1e-12)


def test_iq4_xs_with_unit_sub_scales_is_iq4_nl():
    # ls = 33 on every sub-block: an IQ4_XS super-block equals eight IQ4_NL
    # blocks with the super-block's d
    n, k = 3, 512
    rng = np.random.default_rng(19)
    nb = k // 256
    cb = np.sort(rng.choice(np.arange(-127, 128), 16, replace=False)).astype(np.int8)
    d = rng.uniform(1e-3, 1e-2, (n, nb)).astype(np.float16).astype(np.float64)
    q = rng.integers(0, 16, (n, nb, 256))
    vx = formats.values("iq4_xs", formats.encode("iq4_xs", {"d": d, "ls": np.full((n, nb, 8), 33), "q": q}),
                        n, k, codebook=cb)
    vn = formats.values("iq4_nl", formats.encode("iq4_nl", {"d": np.repeat(d, 8, axis=1),
                                                             "q": q.reshape(n, nb * 8, 32)}), n, k, codebook=cb)
    assert np.array_equal(vx, vn)


def test_exhaustive_q5_k_codes_and_iq4_xs_sub_scales():
    q = (np.arange(256) % 32).reshape(1, 1, 256)
    f = {"d": np.ones((1, 1)), "dmin": np.zeros((1, 1)), "sc": np.ones((1, 1, 8), np.int64),
         "m": np.zeros((1, 1, 8), np.int64), "q": q}
    assert np.array_equal(formats.values("q5_k", formats.encode("q5_k", f), 1, 256)[0], q[0, 0].astype(float))
    ls = np.arange(64).reshape(1, 8, 8)
    cb = np.arange(-8, 8).astype(np.int8)
    raw = formats.encode("iq4_xs", {"d": np.ones((1, 8)), "ls": ls, "q": np.full((1, 8, 256), 9)})
    v = formats.values("iq4_xs", raw, 1, 2048, codebook=cb).reshape(8, 8, 32)
    assert np.array_equal(v[..., 0], (ls[0] - 32).astype(np.float64))


def _sane_scales(raw, fmt, n, k):
    """Overwrite fp16 scale bytes with finite values (random bytes can be NaN)."""
    bb = formats.BLOCK_BYTES[fmt]
    b = raw.reshape(n, -1, bb)
    rng = np.random.default_rng(5)
    offs = [0, 2] if fmt in ("q4_k", "q5_k") else [0]
    for o in offs:
        d = rng.uniform(-4, 4, size=b.shape[:2]).astype(np.float16)
        b[..., o:o + 2] = d.astype("<f2").view(np.uint8).reshape(*b.shape[:2], 2)
    return b.reshape(-1)


@pytest.mark.parametrize("fmt", formats.FORMATS)
def test_bytes_fields_bytes_round_trip(fmt):
    n, k = 5, 512
    rng = np.random.default_rng(1)
    raw = rng.integers(0, 256, n * formats.row_bytes(fmt, k), dtype=np.uint8)
    raw = _sane_scales(raw, fmt, n, k)
    f = formats.decode(fmt, raw, n, k)
    assert np.array_equal(formats.encode(fmt, f), raw)


@pytest.mark.parametrize("fmt", formats.FORMATS)
def test_fields_bytes_fields_round_trip(fmt):
    n, k = 3, 512
    rng = np.random.default_rng(2)
    nb = k // formats.BLOCK_ELEMS[fmt]
    f = {"d": rng.uniform(1e-3, 1e-2, (n, nb)).astype(np.float16).astype(np.float64)}
    if fmt in ("q4_0", "iq4_nl"):
        f["q"] = rng.integers(0, 16, (n, nb, 32))
    elif fmt == "q8_0":
        f["q"] = rng.integers(-128, 128, (n, nb, 32))
    elif fmt in ("q4_k", "q5_k"):
        f["dmin"] = rng.uniform(1e-3, 1e-2, (n, nb)).astype(np.float16).astype(np.float64)
        f["sc"] = rng.integers(0, 64, (n, nb, 8))
        f["m"] = rng.integers(0, 64, (n, nb, 8))
        f["q"] = rng.integers(0, 16 if fmt == "q4_k" else 32, (n, nb, 256))
    elif fmt == "iq4_xs":
        f["ls"] = rng.integers(0, 64, (n, nb, 8))
        f["q"] = rng.integers(0, 16, (n, nb, 256))
    else:
        f["sc"] = rng.integers(-128, 128, (n, nb, 16))
        f["q"] = rng.integers(0, 64, (n, nb, 256))
    g = formats.decode(fmt, formats.encode(fmt, f), n, k)
    for key in f:
        assert np.array_equal(np.asarray(g[key], np.float64), np.asarray(f[key], np.float64)), key


def test_exhaustive_4bit_codes():
    q = np.tile(np.arange(16), 2)[None, None, :]
    for fmt in ("q4_0", "iq4_nl"):
        raw = formats.encode(fmt, {"d": np.ones((1, 1)), "q": q})
        assert np.array_equal(formats.decode(fmt, raw, 1, 32)["q"], q)
    v = formats.values("q4_0", formats.encode("q4_0", {"d": np.ones((1, 1)), "q": q}), 1, 32)
    assert np.array_equal(v[0], np.tile(np.arange(16) - 8, 2))


def test_exhaustive_q4_k_scale_and_min_fields():
    # all 64 values of sc and m, spread over 8 super-blocks
    n, nb = 1, 8
    sc = np.arange(64).reshape(1, 8, 8)
    m = (63 - np.arange(64)).reshape(1, 8, 8)
    q = np.ones((1, nb, 256), np.int64)
    raw = formats.encode("q4_k", {"d": np.ones((1, nb)), "dmin": np.ones((1, nb)), "sc": sc, "m": m, "q": q})
    v = formats.values("q4_k", raw, 1, 256 * nb).reshape(nb, 8, 32)
    assert np.array_equal(v[..., 0], (sc - m)[0].astype(np.float64))


def test_exhaustive_q6_k_codes_and_scales():
    q = np.arange(256).reshape(1, 1, 256) % 64
    sc = (np.arange(16) * 8 - 64).reshape(1, 1, 16)       # -64 .. 56
    raw = formats.encode("q6_k", {"d": np.ones((1, 1)), "sc": sc, "q": q})
    f = formats.decode("q6_k", raw, 1, 256)
    assert np.array_equal(f["q"], q) and np.array_equal(f["sc"], sc)
    allsc = np.arange(-64, 64).reshape(1, 8, 16)
    raw = formats.encode("q6_k", {"d": np.ones((1, 8)), "sc": allsc, "q": np.full((1, 8, 256), 33)})
    v = formats.values("q6_k", raw, 1, 2048).reshape(8, 16, 16)
    assert np.array_equal(v[..., 0], allsc[0].astype(np.float64))
