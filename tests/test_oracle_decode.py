"""Pins of the oracle's weight decoders (CPU only).

Nothing here compares the oracle with a retyped copy of itself: the checks are
the binary16 definition against numpy's float16, exact rational arithmetic on the
logical fields that an independent packer laid into bytes, exhaustive sweeps of
every scale/min/quant value at every sub-block slot, raw-bit layout probes, and a
hand-worked fixture under tests/golden/.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from packer import pack_q4K, pack_q6K, round_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_f16_all_bit_patterns(orc):
    # binary16 -> double for all 65536 encodings, against numpy's float16 type.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))


def _rand_q4K_fields(rng, n, d_scale=2e-3):
    d = (np.abs(rng.standard_normal(n)) * d_scale).astype(np.float16)
    dmin = (np.abs(rng.standard_normal(n)) * d_scale).astype(np.float16)
    sc = rng.integers(0, 64, size=(n, 8))
    mn = rng.integers(0, 64, size=(n, 8))
    q = rng.integers(0, 16, size=(n, 256))
    return d, dmin, sc, mn, q


def test_q4K_exact_rational(orc):
    # Each weight must be the single f32 rounding of the exact d*sc*q - dmin*m.
    rng = np.random.default_rng(11)
    n = 24
    d, dmin, sc, mn, q = _rand_q4K_fields(rng, n)
    # include signs, zero, subnormal and large d/dmin
    d[0], dmin[0] = np.float16(-0.5), np.float16(0.25)
    d[1], dmin[1] = np.float16(0.0), np.float16(-3.0)
    d[2], dmin[2] = np.float16(6e-8), np.float16(6.1e-5)
    d[3], dmin[3] = np.float16(65504.0), np.float16(1e-7)
    raw = pack_q4K(d, dmin, sc, mn, q)
    w = orc.decode(orc.FMT_Q4K, raw, n, 256)
    for b in range(n):
        fd, fm = Fraction(float(d[b])), Fraction(float(dmin[b]))
        for i in range(256):
            j = i // 32
            exact = fd * int(sc[b, j]) * int(q[b, i]) - fm * int(mn[b, j])
            assert w[b, i] == round_to_f32(exact), (b, i)


def test_q4K_sweep_every_scale_min_slot(orc):
    # All 64x64 (scale, min) pairs at each of the 8 sub-block slots, every quant
    # value 0..15 present in each sub-block.  d = 1, dmin = 1/8: the exact value
    # sc*q - m/8 is representable in double, so one rounding to f32 is the answer.
    pairs = np.array([(s, m) for s in range(64) for m in range(64)])
    nb = 8 * len(pairs)
    sc = np.zeros((nb, 8), dtype=np.int64)
    mn = np.zeros((nb, 8), dtype=np.int64)
    rng = np.random.default_rng(5)
    # other slots get random values so that cross-talk between slots shows up
    sc[:] = rng.integers(0, 64, size=(nb, 8))
    mn[:] = rng.integers(0, 64, size=(nb, 8))
    for j in range(8):
        sl = slice(j * len(pairs), (j + 1) * len(pairs))
        sc[sl, j] = pairs[:, 0]
        mn[sl, j] = pairs[:, 1]
    q = np.tile(np.arange(256) % 16, (nb, 1))
    q = (q + rng.integers(0, 16, size=(nb, 1))) % 16  # rotate which quant sits where
    d = np.full(nb, 1.0)
    dmin = np.full(nb, 0.125)
    w = orc.decode(orc.FMT_Q4K, pack_q4K(d, dmin, sc, mn, q), nb, 256)
    j_of_i = np.arange(256) // 32
    exact = sc[:, j_of_i] * q.astype(np.float64) - 0.125 * mn[:, j_of_i]
    assert np.array_equal(w, exact.astype(np.float32))


def test_q4K_textbook_unpack(orc):
    # d = 1, dmin = 0, every scale 1, every min 0 => the decode is the plain quant.
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(4, 256))
    raw = pack_q4K(np.ones(4), np.zeros(4), np.ones((4, 8), int), np.zeros((4, 8), int), q)
    w = orc.decode(orc.FMT_Q4K, raw, 4, 256)
    assert np.array_equal(w, q.astype(np.float32))


def test_q4K_raw_bit_layout(orc):
    # Flip one bit at a time in the raw block and see which logical field moves.
    # Baseline: d = dmin = 1, all scale bytes 0, every quant 1 => w = sc - m = 0.
    def decode_with(scale_bytes, quant_bytes):
        blk = np.zeros((1, 144), dtype=np.uint8)
        blk[0, 0:2] = np.array([1.0], np.float16).view(np.uint8)
        blk[0, 2:4] = np.array([1.0], np.float16).view(np.uint8)
        blk[0, 4:16] = scale_bytes
        blk[0, 16:144] = quant_bytes
        return orc.decode(orc.FMT_Q4K, blk, 1, 256)[0]

    ones = np.full(128, 0x11, dtype=np.uint8)  # every nibble = 1
    # expected (sub-block, 'sc' or 'm', bit) for each of the 96 scale bits
    expect = {}
    for j in range(4):
        for t in range(6):
            expect[(j, t)] = (j, "sc", t)
            expect[(j + 4, t)] = (j, "m", t)
        expect[(j, 6)] = (j + 4, "sc", 4)
        expect[(j, 7)] = (j + 4, "sc", 5)
        expect[(j + 4, 6)] = (j + 4, "m", 4)
        expect[(j + 4, 7)] = (j + 4, "m", 5)
        for t in range(4):
            expect[(j + 8, t)] = (j + 4, "sc", t)
            expect[(j + 8, t + 4)] = (j + 4, "m", t)
    assert len(expect) == 96
    for (byte, bit), (sub, kind, vbit) in expect.items():
        s = np.zeros(12, dtype=np.uint8)
        s[byte] = 1 << bit
        w = decode_with(s, ones)
        want = np.zeros(256, dtype=np.float32)
        want[32 * sub:32 * sub + 32] = (1 << vbit) * (1 if kind == "sc" else -1)
        assert np.array_equal(w, want), (byte, bit)
    # quant positions: byte b, nibble k -> weight 64*(b//32) + 32*k + b%32
    s = np.zeros(12, dtype=np.uint8)
    s[0:4] = 1  # scales of sub-blocks 0..3 = 1
    s[8:12] = 1  # low nibble: scales of sub-blocks 4..7 = 1
    for b in range(128):
        for k in range(2):
            qb = np.zeros(128, dtype=np.uint8)
            qb[b] = 5 << (4 * k)
            w = decode_with(s, qb)
            want = np.zeros(256, dtype=np.float32)
            want[64 * (b // 32) + 32 * k + b % 32] = 5
            assert np.array_equal(w, want), (b, k)


def test_q6K_exact_rational(orc):
    rng = np.random.default_rng(12)
    n = 24
    d = (np.abs(rng.standard_normal(n)) * 1e-3).astype(np.float16)
    d[0], d[1], d[2], d[3] = -2.0, 0.0, 6e-8, 65504.0
    sc = rng.integers(-128, 128, size=(n, 16))
    q = rng.integers(0, 64, size=(n, 256))
    w = orc.decode(orc.FMT_Q6K, pack_q6K(d, sc, q), n, 256)
    for b in range(n):
        fd = Fraction(float(d[b]))
        for i in range(256):
            exact = fd * int(sc[b, i // 16]) * (int(q[b, i]) - 32)
            assert Fraction(float(w[b, i])) == exact, (b, i)  # exact in f32


def test_q6K_sweep_every_scale_slot(orc):
    # Every int8 scale at each of the 16 sub-block slots, every quant 0..63.
    blocks = []
    scs, qs = [], []
    rng = np.random.default_rng(6)
    for j in range(16):
        for s in range(-128, 128):
            for part in range(4):
                sc = rng.integers(-128, 128, size=16)
                sc[j] = s
                q = rng.integers(0, 64, size=256)
                q[16 * j:16 * j + 16] = np.arange(16) + 16 * part
                scs.append(sc)
                qs.append(q)
    sc = np.array(scs)
    q = np.array(qs)
    n = len(sc)
    d = np.full(n, 0.5)
    w = orc.decode(orc.FMT_Q6K, pack_q6K(d, sc, q), n, 256)
    exact = 0.5 * sc[:, np.arange(256) // 16] * (q - 32).astype(np.float64)
    assert np.array_equal(w, exact.astype(np.float32))
    del blocks


def test_q6K_raw_bit_layout(orc):
    # d = 1, all scales 1: w = q - 32.  Set one bit of ql or qh, see which weight moves.
    def dec(ql, qh):
        blk = np.zeros((1, 210), dtype=np.uint8)
        blk[0, 0:128] = ql
        blk[0, 128:192] = qh
        blk[0, 192:208] = 1
        blk[0, 208:210] = np.array([1.0], np.float16).view(np.uint8)
        return orc.decode(orc.FMT_Q6K, blk, 1, 256)[0]

    base = np.full(256, -32.0, dtype=np.float32)
    for byte in range(128):
        for bit in range(8):
            ql = np.zeros(128, np.uint8)
            ql[byte] = 1 << bit
            h, r = divmod(byte, 64)
            c = (r // 32) + (2 if bit >= 4 else 0)
            i = 128 * h + 32 * c + r % 32
            want = base.copy()
            want[i] += 1 << (bit % 4)
            assert np.array_equal(dec(ql, np.zeros(64, np.uint8)), want), (byte, bit)
    for byte in range(64):
        for bit in range(8):
            qh = np.zeros(64, np.uint8)
            qh[byte] = 1 << bit
            h, l = divmod(byte, 32)
            c = bit // 2
            i = 128 * h + 32 * c + l
            want = base.copy()
            want[i] += 1 << (4 + bit % 2)
            assert np.array_equal(dec(np.zeros(128, np.uint8), qh), want), (byte, bit)


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


@pytest.mark.parametrize("name,fmt,N", [("q4K_handworked.txt", 12, 1), ("q6K_handworked.txt", 14, 1)])
def test_handworked_fixture(orc, name, fmt, N):
    fx = _read_fixture(name)
    raw = np.array([int(x, 16) for x in fx["bytes"]], dtype=np.uint8)
    want = np.array([float(x) for x in fx["weights"]], dtype=np.float32)
    got = orc.decode(fmt, raw, N, 256)[0]
    assert np.array_equal(got, want)
