"""Test helpers: an independent block packer and exact-rounding utilities.

The packer goes the other way from the oracle's decoder: it takes the block's
logical fields (d, dmin, 6-bit scales and mins, quants) and lays them into bytes.
It is written from the prose description of the ggml K-quant layouts, not from
the decoder, so a transposed field, a wrong nibble order or a wrong bit position
in either one makes a round trip fail.  (Both follow the same reading of the
layout; parity with ggml's own bytes stays unpinned.)

Layouts, little-endian:
  q4_K (144 B): [0:2] f16 d, [2:4] f16 dmin, [4:16] scale bytes s[0..11],
    [16:144] quant bytes.  For sub-block j < 4: scale in the low 6 bits of s[j],
    min in the low 6 bits of s[j+4].  For j >= 4: the low 4 bits of the scale are
    the low nibble of s[j+4], those of the min its high nibble; the top 2 bits of
    the scale sit in bits 6..7 of s[j-4], those of the min in bits 6..7 of s[j].
    Quants: 64-weight group g uses bytes 32g..32g+31; weight 64g+l (l < 32) is the
    low nibble of byte 32g+l, weight 64g+32+l its high nibble.
  q6_K (210 B): [0:128] ql, [128:192] qh, [192:208] int8 scales, [208:210] f16 d.
    Weight i = 128h + 32c + l: low 4 bits in ql[64h + l + 32(c&1)] (low nibble if
    c < 2, high nibble otherwise), top 2 bits in bits 2c..2c+1 of qh[32h + l];
    scale sc[i // 16]; value d * sc * (q - 32).
  q2_K (84 B): [0:16] one byte per 16-weight sub-block (scale in the low nibble,
    min in the high nibble), [16:80] quant bytes, [80:82] f16 d, [82:84] f16 dmin.
    Weight i = 128h + 32c + l (l < 32) is bits 2c..2c+1 of quant byte 32h + l;
    value d * sc * q - dmin * m for its sub-block i // 16.
  q3_K (110 B): [0:32] high-bit mask, [32:96] 2-bit low parts (placed as q2_K's
    quants), [96:108] scale bytes, [108:110] f16 d.  Weight i = 128h + 32c + l has
    its third bit at bit 4h + c of mask byte l; a set bit means q = low, a clear one
    q = low - 4.  The 16 scales are stored as sc + 32 in 0..63; the low four bits
    of scales 0..3 are the low nibbles of bytes 0..3, of scales 4..7 the low
    nibbles of bytes 4..7, of scales 8..11 the high nibbles of bytes 0..3, of
    scales 12..15 the high nibbles of bytes 4..7; the top two bits of scale
    4g + k are bits 2g..2g+1 of byte 8 + k.  Value d * sc * q.
  q5_K (176 B): [0:16] as q4_K (d, dmin, the same packed scales and mins),
    [16:48] high bits, [48:176] low nibbles placed as q4_K's quants.  Weight
    64g + 32t + l has its fifth bit at bit 2g + t of high-bit byte l.
  q8_K (292 B): [0:4] f32 d, [4:260] int8 q, [260:292] int16 sums of 16 q each.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def f16_bytes(v) -> np.ndarray:
    a = np.asarray(v, dtype=np.float16).reshape(-1)
    return a.view(np.uint8).reshape(-1, 2)


def pack_q4K(d, dmin, sc, mn, q) -> np.ndarray:
    """d, dmin: [n] (cast to f16); sc, mn: int [n, 8] in 0..63; q: int [n, 256] in 0..15."""
    sc = np.asarray(sc, dtype=np.int64)
    mn = np.asarray(mn, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    n = q.shape[0]
    assert sc.shape == (n, 8) and mn.shape == (n, 8) and q.shape == (n, 256)
    assert sc.min() >= 0 and sc.max() < 64 and mn.min() >= 0 and mn.max() < 64
    assert q.min() >= 0 and q.max() < 16
    out = np.zeros((n, 144), dtype=np.uint8)
    out[:, 0:2] = f16_bytes(d)
    out[:, 2:4] = f16_bytes(dmin)
    s = np.zeros((n, 12), dtype=np.int64)
    for j in range(4):
        s[:, j] = (sc[:, j] & 63) | ((sc[:, j + 4] >> 4) << 6)
        s[:, j + 4] = (mn[:, j] & 63) | ((mn[:, j + 4] >> 4) << 6)
        s[:, j + 8] = (sc[:, j + 4] & 15) | ((mn[:, j + 4] & 15) << 4)
    out[:, 4:16] = s.astype(np.uint8)
    qs = np.zeros((n, 128), dtype=np.int64)
    for g in range(4):
        qs[:, 32 * g:32 * g + 32] = q[:, 64 * g:64 * g + 32] | (q[:, 64 * g + 32:64 * g + 64] << 4)
    out[:, 16:144] = qs.astype(np.uint8)
    return out


def pack_q6K(d, sc, q) -> np.ndarray:
    """d: [n] (cast to f16); sc: int [n, 16] in -128..127; q: int [n, 256] in 0..63."""
    sc = np.asarray(sc, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    n = q.shape[0]
    assert sc.shape == (n, 16) and q.shape == (n, 256)
    assert sc.min() >= -128 and sc.max() < 128 and q.min() >= 0 and q.max() < 64
    ql = np.zeros((n, 128), dtype=np.int64)
    qh = np.zeros((n, 64), dtype=np.int64)
    for h in range(2):
        for c in range(4):
            for l in range(32):
                i = 128 * h + 32 * c + l
                low, high = q[:, i] & 15, q[:, i] >> 4
                ql[:, 64 * h + l + 32 * (c & 1)] |= low << (4 if c >= 2 else 0)
                qh[:, 32 * h + l] |= high << (2 * c)
    out = np.zeros((n, 210), dtype=np.uint8)
    out[:, 0:128] = ql.astype(np.uint8)
    out[:, 128:192] = qh.astype(np.uint8)
    out[:, 192:208] = sc.astype(np.int8).view(np.uint8)
    out[:, 208:210] = f16_bytes(d)
    return out


def pack_q2K(d, dmin, sc, mn, q) -> np.ndarray:
    """d, dmin: [n] (cast to f16); sc, mn: int [n, 16] in 0..15; q: int [n, 256] in 0..3."""
    sc = np.asarray(sc, dtype=np.int64)
    mn = np.asarray(mn, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    n = q.shape[0]
    assert sc.shape == (n, 16) and mn.shape == (n, 16) and q.shape == (n, 256)
    assert sc.min() >= 0 and sc.max() < 16 and mn.min() >= 0 and mn.max() < 16
    assert q.min() >= 0 and q.max() < 4
    out = np.zeros((n, 84), dtype=np.uint8)
    out[:, 0:16] = (sc | (mn << 4)).astype(np.uint8)
    qs = np.zeros((n, 64), dtype=np.int64)
    for h in range(2):
        for c in range(4):
            qs[:, 32 * h:32 * h + 32] |= q[:, 128 * h + 32 * c:128 * h + 32 * c + 32] << (2 * c)
    out[:, 16:80] = qs.astype(np.uint8)
    out[:, 80:82] = f16_bytes(d)
    out[:, 82:84] = f16_bytes(dmin)
    return out


def pack_q3K(d, sc, q) -> np.ndarray:
    """d: [n] (cast to f16); sc: int [n, 16] in -32..31; q: int [n, 256] in -4..3."""
    sc = np.asarray(sc, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    n = q.shape[0]
    assert sc.shape == (n, 16) and q.shape == (n, 256)
    assert sc.min() >= -32 and sc.max() < 32 and q.min() >= -4 and q.max() < 4
    hm = np.zeros((n, 32), dtype=np.int64)
    qs = np.zeros((n, 64), dtype=np.int64)
    for h in range(2):
        for c in range(4):
            blk = q[:, 128 * h + 32 * c:128 * h + 32 * c + 32]
            hm |= (blk >= 0).astype(np.int64) << (4 * h + c)
            qs[:, 32 * h:32 * h + 32] |= np.where(blk >= 0, blk, blk + 4) << (2 * c)
    u = sc + 32
    sb = np.zeros((n, 12), dtype=np.int64)
    for k in range(4):
        sb[:, k] = (u[:, k] & 15) | ((u[:, 8 + k] & 15) << 4)
        sb[:, 4 + k] = (u[:, 4 + k] & 15) | ((u[:, 12 + k] & 15) << 4)
        sb[:, 8 + k] = ((u[:, k] >> 4) | ((u[:, 4 + k] >> 4) << 2) | ((u[:, 8 + k] >> 4) << 4)
                        | ((u[:, 12 + k] >> 4) << 6))
    out = np.zeros((n, 110), dtype=np.uint8)
    out[:, 0:32] = hm.astype(np.uint8)
    out[:, 32:96] = qs.astype(np.uint8)
    out[:, 96:108] = sb.astype(np.uint8)
    out[:, 108:110] = f16_bytes(d)
    return out


def pack_q5K(d, dmin, sc, mn, q) -> np.ndarray:
    """d, dmin: [n] (cast to f16); sc, mn: int [n, 8] in 0..63; q: int [n, 256] in 0..31."""
    q = np.asarray(q, dtype=np.int64)
    n = q.shape[0]
    assert q.shape == (n, 256) and q.min() >= 0 and q.max() < 32
    low = pack_q4K(d, dmin, sc, mn, q & 15)  # header and low nibbles, laid out as q4_K
    qh = np.zeros((n, 32), dtype=np.int64)
    for g in range(4):
        for t in range(2):
            qh |= (q[:, 64 * g + 32 * t:64 * g + 32 * t + 32] >> 4) << (2 * g + t)
    out = np.zeros((n, 176), dtype=np.uint8)
    out[:, 0:16] = low[:, 0:16]
    out[:, 16:48] = qh.astype(np.uint8)
    out[:, 48:176] = low[:, 16:144]
    return out


def q8K_fields(blocks: np.ndarray):
    """Split q8_K bytes [..., 292] into (d f32 [...], q int8 [..., 256], sums int16 [..., 16])."""
    b = np.ascontiguousarray(blocks).reshape(-1, 292)
    d = b[:, 0:4].copy().view(np.float32).reshape(-1)
    q = b[:, 4:260].copy().view(np.int8)
    s = b[:, 260:292].copy().view(np.int16)
    return d, q, s


def frac_of(v) -> Fraction:
    return Fraction(float(v))


def round_to_f32(x: Fraction) -> np.float32:
    """The f32 nearest to the exact rational x, ties to even (single rounding)."""
    c = np.float32(float(x))  # within one f32 ulp of x
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        err = abs(Fraction(float(cand)) - x)
        if best is None or err < best[0] or (
                err == best[0] and (int(np.float32(cand).view(np.uint32)) & 1) == 0):
            best = (err, np.float32(cand))
    return best[1]
