"""Pins of the oracle's q2_K, q3_K and q5_K decoders (CPU only).

The same kinds of check as for q4_K and q6_K, none of them a retyped copy of
the decoder: exact rational arithmetic on logical fields that the independent
packer (tests/packer.py) laid into bytes, exhaustive sweeps of every scale (and
min) value at every sub-block slot with every quant value present, one-bit
probes of every raw bit against the layout written out below, and hand-worked
blocks under tests/golden/.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from packer import pack_q2K, pack_q3K, pack_q5K, round_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
Q2, Q3, Q5 = 10, 11, 13


def _special_d(d, dmin=None):
    d[0], d[1], d[2], d[3] = -0.5, 0.0, 6e-8, 65504.0
    if dmin is not None:
        dmin[0], dmin[1], dmin[2], dmin[3] = 0.25, -3.0, 6.1e-5, 1e-7


# ---------------------------------------------------------------- exact values

def test_q2K_exact_rational(orc):
    rng = np.random.default_rng(21)
    n = 24
    d = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    dmin = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    _special_d(d, dmin)
    sc = rng.integers(0, 16, size=(n, 16))
    mn = rng.integers(0, 16, size=(n, 16))
    q = rng.integers(0, 4, size=(n, 256))
    w = orc.decode(Q2, pack_q2K(d, dmin, sc, mn, q), n, 256)
    for b in range(n):
        fd, fm = Fraction(float(d[b])), Fraction(float(dmin[b]))
        for i in range(256):
            exact = fd * int(sc[b, i // 16]) * int(q[b, i]) - fm * int(mn[b, i // 16])
            assert w[b, i] == round_to_f32(exact), (b, i)


def test_q3K_exact_rational(orc):
    rng = np.random.default_rng(22)
    n = 24
    d = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    _special_d(d)
    sc = rng.integers(-32, 32, size=(n, 16))
    q = rng.integers(-4, 4, size=(n, 256))
    w = orc.decode(Q3, pack_q3K(d, sc, q), n, 256)
    for b in range(n):
        fd = Fraction(float(d[b]))
        for i in range(256):
            exact = fd * int(sc[b, i // 16]) * int(q[b, i])
            assert Fraction(float(w[b, i])) == exact, (b, i)  # exact in f32


def test_q5K_exact_rational(orc):
    rng = np.random.default_rng(23)
    n = 24
    d = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    dmin = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    _special_d(d, dmin)
    sc = rng.integers(0, 64, size=(n, 8))
    mn = rng.integers(0, 64, size=(n, 8))
    q = rng.integers(0, 32, size=(n, 256))
    w = orc.decode(Q5, pack_q5K(d, dmin, sc, mn, q), n, 256)
    for b in range(n):
        fd, fm = Fraction(float(d[b])), Fraction(float(dmin[b]))
        for i in range(256):
            exact = fd * int(sc[b, i // 32]) * int(q[b, i]) - fm * int(mn[b, i // 32])
            assert w[b, i] == round_to_f32(exact), (b, i)


# ---------------------------------------------------------------- sweeps

def test_q2K_sweep_every_scale_min_slot(orc):
    # all 16 x 16 (scale, min) pairs at each of the 16 slots; every quant 0..3 in
    # each sub-block; d = 1, dmin = 1/4: sc*q - m/4 is exact in f32
    rng = np.random.default_rng(31)
    pairs = np.array([(s, m) for s in range(16) for m in range(16)])
    nb = 16 * len(pairs)
    sc = rng.integers(0, 16, size=(nb, 16))
    mn = rng.integers(0, 16, size=(nb, 16))
    for j in range(16):
        sl = slice(j * len(pairs), (j + 1) * len(pairs))
        sc[sl, j] = pairs[:, 0]
        mn[sl, j] = pairs[:, 1]
    q = (np.tile(np.arange(256) % 4, (nb, 1)) + rng.integers(0, 4, size=(nb, 1))) % 4
    w = orc.decode(Q2, pack_q2K(np.ones(nb), np.full(nb, 0.25), sc, mn, q), nb, 256)
    j_of_i = np.arange(256) // 16
    exact = sc[:, j_of_i] * q.astype(np.float64) - 0.25 * mn[:, j_of_i]
    assert np.array_equal(w, exact.astype(np.float32))


def test_q3K_sweep_every_scale_slot(orc):
    # every scale -32..31 at each of the 16 slots; every quant -4..3 in each sub-block
    rng = np.random.default_rng(32)
    rows_sc, rows_q = [], []
    for j in range(16):
        for s in range(-32, 32):
            for part in range(2):
                sc = rng.integers(-32, 32, size=16)
                sc[j] = s
                q = rng.integers(-4, 4, size=256)
                q[16 * j:16 * j + 16] = (np.arange(16) + 8 * part) % 8 - 4
                rows_sc.append(sc)
                rows_q.append(q)
    sc, q = np.array(rows_sc), np.array(rows_q)
    n = len(sc)
    w = orc.decode(Q3, pack_q3K(np.full(n, 0.5), sc, q), n, 256)
    exact = 0.5 * sc[:, np.arange(256) // 16] * q.astype(np.float64)
    assert np.array_equal(w, exact.astype(np.float32))


def test_q5K_sweep_every_scale_min_slot(orc):
    rng = np.random.default_rng(33)
    pairs = np.array([(s, m) for s in range(64) for m in range(64)])
    nb = 8 * len(pairs)
    sc = rng.integers(0, 64, size=(nb, 8))
    mn = rng.integers(0, 64, size=(nb, 8))
    for j in range(8):
        sl = slice(j * len(pairs), (j + 1) * len(pairs))
        sc[sl, j] = pairs[:, 0]
        mn[sl, j] = pairs[:, 1]
    q = (np.tile(np.arange(256) % 32, (nb, 1)) + rng.integers(0, 32, size=(nb, 1))) % 32
    w = orc.decode(Q5, pack_q5K(np.ones(nb), np.full(nb, 0.125), sc, mn, q), nb, 256)
    j_of_i = np.arange(256) // 32
    exact = sc[:, j_of_i] * q.astype(np.float64) - 0.125 * mn[:, j_of_i]
    assert np.array_equal(w, exact.astype(np.float32))


# ---------------------------------------------------------------- raw bits

def _f16(v):
    return np.array([v], np.float16).view(np.uint8)


def test_q2K_raw_bit_layout(orc):
    def dec(scales, qs):
        blk = np.zeros((1, 84), np.uint8)
        blk[0, 0:16] = scales
        blk[0, 16:80] = qs
        blk[0, 80:82] = _f16(1.0)
        blk[0, 82:84] = _f16(1.0)
        return orc.decode(Q2, blk, 1, 256)[0]

    # scale/min bits, every quant 1: w = sc - m
    for j in range(16):
        for t in range(8):
            s = np.zeros(16, np.uint8)
            s[j] = 1 << t
            want = np.zeros(256, np.float32)
            want[16 * j:16 * j + 16] = (1 << t) if t < 4 else -(1 << (t - 4))
            assert np.array_equal(dec(s, np.full(64, 0x55, np.uint8)), want), (j, t)
    # quant bits, every scale 1 and min 0: w = q.  byte 32h + l, bit t -> weight
    # 128h + 32(t // 2) + l, value 2^(t % 2)
    for b in range(64):
        for t in range(8):
            qs = np.zeros(64, np.uint8)
            qs[b] = 1 << t
            h, l = divmod(b, 32)
            want = np.zeros(256, np.float32)
            want[128 * h + 32 * (t // 2) + l] = 1 << (t % 2)
            assert np.array_equal(dec(np.ones(16, np.uint8), qs), want), (b, t)


def test_q3K_raw_bit_layout(orc):
    def dec(hm, qs, scales):
        blk = np.zeros((1, 110), np.uint8)
        blk[0, 0:32] = hm
        blk[0, 32:96] = qs
        blk[0, 96:108] = scales
        blk[0, 108:110] = _f16(1.0)
        return orc.decode(Q3, blk, 1, 256)[0]

    # scale stored 33 everywhere (sc = 1): low nibbles 1 in bytes 0..7, top bits
    # 2 in bytes 8..11 (binary 10 in every 2-bit field)
    one = np.array([0x11] * 8 + [0xAA] * 4, np.uint8)
    # mask bits, low parts 0: w = -4, or 0 where the bit is set.  Byte l, bit t ->
    # weight 128(t // 4) + 32(t % 4) + l
    for l in range(32):
        for t in range(8):
            hm = np.zeros(32, np.uint8)
            hm[l] = 1 << t
            want = np.full(256, -4.0, np.float32)
            want[128 * (t // 4) + 32 * (t % 4) + l] = 0.0
            assert np.array_equal(dec(hm, np.zeros(64, np.uint8), one), want), (l, t)
    # low-part bits, mask all set (q = low): placed as q2_K's quants
    for b in range(64):
        for t in range(8):
            qs = np.zeros(64, np.uint8)
            qs[b] = 1 << t
            h, l = divmod(b, 32)
            want = np.zeros(256, np.float32)
            want[128 * h + 32 * (t // 2) + l] = 1 << (t % 2)
            assert np.array_equal(dec(np.full(32, 0xFF, np.uint8), qs, one), want), (b, t)
    # scale bits, every q = 1 (mask set, low parts 01): w = stored scale - 32;
    # baseline all scale bytes 0 -> w = -32 everywhere
    ones_q = np.full(64, 0x55, np.uint8)
    for byte in range(12):
        for t in range(8):
            s = np.zeros(12, np.uint8)
            s[byte] = 1 << t
            if byte < 8:
                k, hi = byte % 4, byte // 4  # bytes 4..7 hold scales 4..7 / 12..15
                j = (k + 4 * hi) + (8 if t >= 4 else 0)
                add = 1 << (t % 4)
            else:
                k = byte - 8
                j = 4 * (t // 2) + k
                add = 16 << (t % 2)
            want = np.full(256, -32.0, np.float32)
            want[16 * j:16 * j + 16] += add
            assert np.array_equal(dec(np.full(32, 0xFF, np.uint8), ones_q, s), want), (byte, t)


def test_q5K_raw_bit_layout(orc):
    def dec(scales, qh, qs):
        blk = np.zeros((1, 176), np.uint8)
        blk[0, 0:2] = _f16(1.0)
        blk[0, 2:4] = _f16(1.0)
        blk[0, 4:16] = scales
        blk[0, 16:48] = qh
        blk[0, 48:176] = qs
        return orc.decode(Q5, blk, 1, 256)[0]

    s = np.zeros(12, np.uint8)
    s[0:4] = 1
    s[8:12] = 1  # every scale 1, every min 0: w = q
    # high bits: byte l, bit t -> weight 64(t // 2) + 32(t % 2) + l, value 16
    for l in range(32):
        for t in range(8):
            qh = np.zeros(32, np.uint8)
            qh[l] = 1 << t
            want = np.zeros(256, np.float32)
            want[64 * (t // 2) + 32 * (t % 2) + l] = 16
            assert np.array_equal(dec(s, qh, np.zeros(128, np.uint8)), want), (l, t)
    # low nibbles: byte b, nibble k -> weight 64(b // 32) + 32k + b % 32
    for b in range(128):
        for k in range(2):
            qs = np.zeros(128, np.uint8)
            qs[b] = 5 << (4 * k)
            want = np.zeros(256, np.float32)
            want[64 * (b // 32) + 32 * k + b % 32] = 5
            assert np.array_equal(dec(s, np.zeros(32, np.uint8), qs), want), (b, k)
    # the 96 scale/min bits sit where q4_K's do: every quant 1 -> w = sc - m
    for byte in range(12):
        for bit in range(8):
            sb = np.zeros(12, np.uint8)
            sb[byte] = 1 << bit
            if byte < 4:
                sub, kind, v = (byte, "sc", bit) if bit < 6 else (byte + 4, "sc", bit - 2)
            elif byte < 8:
                sub, kind, v = (byte - 4, "m", bit) if bit < 6 else (byte, "m", bit - 2)
            else:
                sub, kind, v = (byte - 4, "sc", bit) if bit < 4 else (byte - 4, "m", bit - 4)
            want = np.zeros(256, np.float32)
            want[32 * sub:32 * sub + 32] = (1 << v) * (1 if kind == "sc" else -1)
            assert np.array_equal(dec(sb, np.zeros(32, np.uint8), np.full(128, 0x11, np.uint8)),
                                  want), (byte, bit)


# ---------------------------------------------------------------- textbook cases

@pytest.mark.parametrize("fmt", [Q2, Q5])
def test_plain_quant_when_scales_are_one(orc, fmt):
    # d = 1, dmin = 0, unit scales, zero mins: the decode is the plain quant
    rng = np.random.default_rng(fmt)
    if fmt == Q2:
        q = rng.integers(0, 4, size=(4, 256))
        raw = pack_q2K(np.ones(4), np.zeros(4), np.ones((4, 16), int), np.zeros((4, 16), int), q)
    else:
        q = rng.integers(0, 32, size=(4, 256))
        raw = pack_q5K(np.ones(4), np.zeros(4), np.ones((4, 8), int), np.zeros((4, 8), int), q)
    assert np.array_equal(orc.decode(fmt, raw, 4, 256), q.astype(np.float32))


def test_q3K_plain_quant_when_scales_are_one(orc):
    rng = np.random.default_rng(3)
    q = rng.integers(-4, 4, size=(4, 256))
    raw = pack_q3K(np.ones(4), np.ones((4, 16), int), q)
    assert np.array_equal(orc.decode(Q3, raw, 4, 256), q.astype(np.float32))


def test_unknown_formats_refused(orc):
    raw = np.zeros(210, np.uint8)
    out = np.zeros(256, np.float32)
    for fmt in (-1, 0, 8, 9, 15, 16):
        assert orc.load().oracle_decode(fmt, raw.ctypes.data, 1, out.ctypes.data) == -1


# ---------------------------------------------------------------- hand-worked

def _read_fixture(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            rows[key.strip()] = val.split()
    return rows


@pytest.mark.parametrize("name,fmt", [("q2K_handworked.txt", Q2), ("q3K_handworked.txt", Q3),
                                      ("q5K_handworked.txt", Q5)])
def test_handworked_fixture(orc, name, fmt):
    fx = _read_fixture(name)
    raw = np.array([int(x, 16) for x in fx["bytes"]], dtype=np.uint8)
    want = np.array([float(x) for x in fx["weights"]], dtype=np.float32)
    assert np.array_equal(orc.decode(fmt, raw, 1, 256)[0], want)
