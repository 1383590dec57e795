"""The seven block formats: byte layout, decode and encode (oracle side).

Value formulas are those of the decode-GEMV workloads:
  Q4_0    value = d * (q - 8),          q in 0..15, 32-element blocks
  Q8_0    value = d * q,                q in -127..127, 32-element blocks
  IQ4_NL  value = d * cb[q],            q in 0..15 indexing a sorted int8[16]
  Q4_K    value = d * sc_j * q - dmin * m_j, q in 0..15, 256-element
          super-blocks of eight 32-element sub-blocks j with 6-bit sc_j, m_j
  Q6_K    value = d * sc_j * (q - 32),  q in 0..63, 256-element super-blocks
          of sixteen 16-element sub-blocks j with int8 sc_j
  Q5_K    value = d * sc_j * q - dmin * m_j, q in 0..31 (Q4_K with a fifth
          code bit), 256-element super-blocks
  IQ4_XS  value = d * (ls_j - 32) * cb[q], q in 0..15 indexing the IQ4_NL
          codebook, 256-element super-blocks of eight 32-element sub-blocks
          with 6-bit unsigned sub-scales ls_j
The last two are the formats whose single-matrix bandwidth the pages report
("Why expert caching can't save dense models", xhh.club, summary of the
measurements: IQ4_XS, Q5_K and Q6_K matrices); the pages name them but give
no field layout, so theirs below is this library's own reading.
The method reads these blocks in place, with the correction terms of the
K-quant super-blocks and a small codebook for the non-linear 4-bit format
("Why expert caching can't save dense models", xhh.club, Q&A on computing
GGUF blocks without FP16 expansion).

The pages do not give the byte order inside a block. The reading used here
(and by the GPU kernels, written separately) is, little-endian throughout:

  Q4_0 / IQ4_NL (18 B): bytes 0-1 d (fp16); bytes 2..17 = qs[16].
      Element i < 16 is the low nibble of qs[i]; element i >= 16 is the high
      nibble of qs[i - 16].
  Q8_0 (34 B): bytes 0-1 d; bytes 2..33 the 32 int8 codes in element order.
  Q4_K (144 B): bytes 0-1 d, 2-3 dmin; bytes 4..15 = scales[12], read as one
      96-bit little-endian integer holding sixteen 6-bit fields, field f at
      bits 6f..6f+5: fields 0..7 are sc_0..sc_7, fields 8..15 are m_0..m_7;
      bytes 16..143 = qs[128], sub-block j's 32 codes in qs[16j..16j+15] with
      the Q4_0 nibble order.
  Q6_K (210 B): bytes 0-1 d; bytes 2..17 sc[16] (int8); bytes 18..145
      ql[128]; bytes 146..209 qh[64]. Element e = 32g + i (g = 0..7,
      i = 0..31): low 4 bits from ql[16g + (i mod 16)] (low nibble if i < 16,
      else high nibble); high 2 bits are bits 2*(i div 8) and 2*(i div 8)+1 of
      qh[8g + (i mod 8)]; q = low | high << 4; sub-block j = e div 16.
  Q5_K (176 B): bytes 0-1 d, 2-3 dmin, 4..15 scales[12] as in Q4_K;
      bytes 16..47 = qh[32]; bytes 48..175 = qs[128] with Q4_K's sub-block
      and nibble order for the low 4 bits. The fifth bit of element
      e = 32j + i (i = 0..31) is bit (i div 4) of qh[4j + (i mod 4)], i.e.
      sub-block j's 32 fifth bits form the little-endian word qh[4j..4j+3]
      with element i at bit 8 (i mod 4) + (i div 4); q = low | fifth << 4.
  IQ4_XS (136 B): bytes 0-1 d; bytes 2-3 scales_h (uint16); bytes 4..7
      scales_l[4]; bytes 8..135 qs[128] with Q4_K's sub-block and nibble
      order. Sub-scale ls_j (0..63) = low 4 bits from scales_l[j div 2]
      (low nibble for even j) | bits 2j, 2j+1 of scales_h as bits 4, 5.
"""
from __future__ import annotations

import numpy as np

BLOCK_ELEMS = {"q4_0": 32, "q8_0": 32, "iq4_nl": 32, "q4_k": 256, "q6_k": 256, "q5_k": 256,
               "iq4_xs": 256}
BLOCK_BYTES = {"q4_0": 18, "q8_0": 34, "iq4_nl": 18, "q4_k": 144, "q6_k": 210, "q5_k": 176,
               "iq4_xs": 136}
CODEBOOK_FORMATS = ("iq4_nl", "iq4_xs")
FORMATS = tuple(BLOCK_BYTES)


def row_bytes(fmt, k):
    be = BLOCK_ELEMS[fmt]
    if k <= 0 or k % be:
        raise ValueError(f"{fmt}: K={k} must be a positive multiple of {be}")
    return k // be * BLOCK_BYTES[fmt]


def _blocks(fmt, raw, n, k):
    raw = np.asarray(raw, dtype=np.uint8).reshape(-1)
    need = n * row_bytes(fmt, k)
    if raw.size < need:
        raise ValueError("weight buffer too small")
    return raw[:need].reshape(n, k // BLOCK_ELEMS[fmt], BLOCK_BYTES[fmt])


def _fp16(b, off):
    return b[..., off:off + 2].copy().view("<f2")[..., 0].astype(np.float64)


def _nibbles32(qs):
    """qs[..., 16] bytes -> 32 codes: low nibbles first, then high nibbles."""
    qs = qs.astype(np.int64)
    return np.concatenate([qs & 0xF, qs >> 4], axis=-1)


def _pack_nibbles32(q):
    q = np.asarray(q, np.int64)
    return (q[..., :16] | (q[..., 16:] << 4)).astype(np.uint8)


# ---------------------------------------------------------------- decode ---

def decode(fmt, raw, n, k, codebook=None):
    """Decode packed bytes to a dict of fields (float64 scales, int64 codes).

    Shapes: nb = blocks per row.
      q4_0 / iq4_nl: d[n, nb], q[n, nb, 32]
      q8_0:          d[n, nb], q[n, nb, 32]
      q4_k / q5_k:   d[n, nb], dmin[n, nb], sc[n, nb, 8], m[n, nb, 8], q[n, nb, 256]
      q6_k:          d[n, nb], sc[n, nb, 16], q[n, nb, 256]
      iq4_xs:        d[n, nb], ls[n, nb, 8], q[n, nb, 256]
    """
    b = _blocks(fmt, raw, n, k)
    if fmt in ("q4_0", "iq4_nl"):
        return {"d": _fp16(b, 0), "q": _nibbles32(b[..., 2:18])}
    if fmt == "q8_0":
        return {"d": _fp16(b, 0), "q": b[..., 2:34].view(np.int8).astype(np.int64)}
    if fmt in ("q4_k", "q5_k"):
        bits = np.unpackbits(b[..., 4:16], axis=-1, bitorder="little")      # [.., 96]
        fields = (bits.reshape(*bits.shape[:-1], 16, 6).astype(np.int64)
                  * (1 << np.arange(6))).sum(-1)                             # [.., 16]
        q0 = 16 if fmt == "q4_k" else 48
        qs = b[..., q0:q0 + 128].reshape(n, -1, 8, 16)
        q = _nibbles32(qs)                                                   # [n, nb, 8, 32]
        if fmt == "q5_k":
            qh = b[..., 16:48].reshape(n, -1, 8, 4).astype(np.int64)         # [n, nb, 8, 4]
            i = np.arange(32)
            fifth = (qh[..., i % 4] >> (i // 4)) & 1                         # [n, nb, 8, 32]
            q = q | (fifth << 4)
        return {"d": _fp16(b, 0), "dmin": _fp16(b, 2), "sc": fields[..., :8],
                "m": fields[..., 8:], "q": q.reshape(n, -1, 256)}
    if fmt == "iq4_xs":
        sh = b[..., 2:4].copy().view("<u2")[..., 0].astype(np.int64)        # [n, nb]
        sl = b[..., 4:8].astype(np.int64)                                    # [n, nb, 4]
        j = np.arange(8)
        ls = ((sl[..., j // 2] >> (4 * (j % 2))) & 0xF) | (((sh[..., None] >> (2 * j)) & 3) << 4)
        q = _nibbles32(b[..., 8:136].reshape(n, -1, 8, 16)).reshape(n, -1, 256)
        return {"d": _fp16(b, 0), "ls": ls, "q": q}
    if fmt == "q6_k":
        sc = b[..., 2:18].view(np.int8).astype(np.int64)
        ql = b[..., 18:146].astype(np.int64)
        qh = b[..., 146:210].astype(np.int64)
        g = np.arange(8)[:, None]
        i = np.arange(32)[None, :]
        lo_idx = 16 * g + (i % 16)                       # [8, 32]
        lo = ql[..., lo_idx]
        lo = np.where(i < 16, lo & 0xF, lo >> 4)
        hi = (qh[..., 8 * g + (i % 8)] >> (2 * (i // 8))) & 3
        q = (lo | (hi << 4)).reshape(n, -1, 256)
        return {"d": _fp16(b, 0), "sc": sc, "q": q}
    raise ValueError(fmt)


def values(fmt, raw, n, k, codebook=None):
    """Dequantized weights W_hat[n, k] in float64 (each value exact)."""
    f = decode(fmt, raw, n, k)
    if fmt == "q4_0":
        v = f["d"][..., None] * (f["q"] - 8)
    elif fmt == "q8_0":
        v = f["d"][..., None] * f["q"]
    elif fmt == "iq4_nl":
        cb = np.asarray(codebook, np.int64)
        v = f["d"][..., None] * cb[f["q"]]
    elif fmt in ("q4_k", "q5_k"):
        q = f["q"].reshape(n, -1, 8, 32)
        v = (f["d"][..., None, None] * f["sc"][..., None] * q
             - f["dmin"][..., None, None] * f["m"][..., None])
    elif fmt == "iq4_xs":
        cb = np.asarray(codebook, np.int64)
        q = f["q"].reshape(n, -1, 8, 32)
        v = f["d"][..., None, None] * (f["ls"][..., None] - 32) * cb[q]
    elif fmt == "q6_k":
        q = f["q"].reshape(n, -1, 16, 16)
        v = f["d"][..., None, None] * f["sc"][..., None] * (q - 32)
    else:
        raise ValueError(fmt)
    return v.reshape(n, k).astype(np.float64)


# ---------------------------------------------------------------- encode ---

def encode(fmt, fields):
    """Inverse of `decode`: fields (same shapes) -> uint8[n * row_bytes].

    Scales are given as float64/float16 and stored as fp16 (they must be
    representable for an exact round trip)."""
    d = np.asarray(fields["d"]).astype(np.float16)
    n, nb = d.shape
    out = np.zeros((n, nb, BLOCK_BYTES[fmt]), np.uint8)
    out[..., 0:2] = d.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    q = np.asarray(fields["q"], np.int64)
    if fmt in ("q4_0", "iq4_nl"):
        out[..., 2:18] = _pack_nibbles32(q)
    elif fmt == "q8_0":
        out[..., 2:34] = q.astype(np.int8).view(np.uint8)
    elif fmt in ("q4_k", "q5_k"):
        dm = np.asarray(fields["dmin"]).astype(np.float16)
        out[..., 2:4] = dm.astype("<f2").view(np.uint8).reshape(n, nb, 2)
        f16 = np.concatenate([np.asarray(fields["sc"], np.int64),
                              np.asarray(fields["m"], np.int64)], axis=-1)   # [n, nb, 16]
        bits = ((f16[..., None] >> np.arange(6)) & 1).reshape(n, nb, 96).astype(np.uint8)
        out[..., 4:16] = np.packbits(bits, axis=-1, bitorder="little")
        qg = q.reshape(n, nb, 8, 32)
        q0 = 16 if fmt == "q4_k" else 48
        out[..., q0:q0 + 128] = _pack_nibbles32(qg & 0xF).reshape(n, nb, 128)
        if fmt == "q5_k":
            fifth = qg >> 4                                                  # [n, nb, 8, 32]
            qh = np.zeros((n, nb, 8, 4), np.int64)
            for i in range(32):
                qh[..., i % 4] |= fifth[..., i] << (i // 4)
            out[..., 16:48] = qh.reshape(n, nb, 32).astype(np.uint8)
    elif fmt == "iq4_xs":
        ls = np.asarray(fields["ls"], np.int64)                              # [n, nb, 8]
        sh = np.zeros((n, nb), np.int64)
        sl = np.zeros((n, nb, 4), np.int64)
        for j in range(8):
            sh |= (ls[..., j] >> 4) << (2 * j)
            sl[..., j // 2] |= (ls[..., j] & 0xF) << (4 * (j % 2))
        out[..., 2:4] = sh.astype("<u2").view(np.uint8).reshape(n, nb, 2)
        out[..., 4:8] = sl.astype(np.uint8)
        out[..., 8:136] = _pack_nibbles32(q.reshape(n, nb, 8, 32)).reshape(n, nb, 128)
    elif fmt == "q6_k":
        out[..., 2:18] = np.asarray(fields["sc"], np.int64).astype(np.int8).view(np.uint8)
        qg = q.reshape(n, nb, 8, 32)
        lo = qg & 0xF
        hi = qg >> 4
        ql = lo[..., :16] | (lo[..., 16:] << 4)                       # [n, nb, 8, 16]
        out[..., 18:146] = ql.reshape(n, nb, 128).astype(np.uint8)
        qh = np.zeros((n, nb, 8, 8), np.int64)
        for t in range(4):                                             # i div 8
            qh |= hi[..., 8 * t:8 * t + 8] << (2 * t)
        out[..., 146:210] = qh.reshape(n, nb, 64).astype(np.uint8)
    else:
        raise ValueError(fmt)
    return out.reshape(-1)
