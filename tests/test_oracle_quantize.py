"""Pins of the oracle's q8_K activation quantizer (CPU only).

The quantizer reading: per 256-block, d = amax/127 in f32, q = round-half-even of
x/d clamped to [-127, 127], sums over groups of 16 (molayo article, status row
"src/ -- C++ engine": activations are quantized to int8 blocks the way llama.cpp
does; the formula itself is a reading of that sentence, which names no formula).  The checks are properties the
definition fixes: the error bound of rounding, the extreme code, exact ties,
reachability of every code, odd symmetry, power-of-two scale invariance, the group
sums and the zero block.
"""
import numpy as np

from packer import q8K_fields


def _rand(rng, M, K, outliers=True):
    x = rng.standard_normal((M, K)).astype(np.float32)
    if outliers:
        x[:, rng.choice(K, 4, replace=False)] *= 20
    return x


def test_shape_and_error_bound(orc):
    rng = np.random.default_rng(1)
    x = _rand(rng, 7, 1024)
    xq = orc.quantize_q8K(x)
    assert xq.shape == (7, 4 * 292)
    d, q, s = q8K_fields(xq)
    xb = x.reshape(-1, 256).astype(np.float64)
    dd = d.astype(np.float64)[:, None]
    # |x - d*q| <= d/2 up to the f32 rounding of x/d (relative 2^-24 of 127)
    err = np.abs(xb - dd * q)
    assert np.all(err <= dd * (0.5 + 127 * 2.0 ** -23))
    # the largest magnitude maps to +-127 and nothing exceeds 127 in magnitude
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert q.min() >= -127
    # d is the f32 division amax/127
    amax = np.abs(x.reshape(-1, 256)).max(axis=1)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float32))
    # group sums
    assert np.array_equal(s.astype(np.int64), q.reshape(-1, 16, 16).astype(np.int64).sum(axis=2))


def test_exact_ties_round_half_even(orc):
    # amax = 127 * 2^-7 makes d = 2^-7 exactly; x = (k + 1/2) * 2^-7 then divides to
    # exactly k + 1/2, which must go to the even neighbour.
    ks = np.arange(-127, 127)  # k + 1/2 in [-126.5, 126.5]
    x = np.zeros((1, 512), dtype=np.float32)
    x[0, 0] = 127 * 2.0 ** -7
    x[0, 1:1 + len(ks)] = (ks + 0.5) * 2.0 ** -7
    x[0, 256] = -127 * 2.0 ** -7
    x[0, 257:257 + len(ks)] = (ks + 0.5) * 2.0 ** -7
    d, q, _ = q8K_fields(orc.quantize_q8K(x))
    assert np.all(d == np.float32(2.0 ** -7))
    want = np.where(ks % 2 == 0, ks, ks + 1)  # k even -> k, k odd -> k+1 (even)
    assert np.array_equal(q[0, 1:1 + len(ks)], want)
    assert np.array_equal(q[1, 1:1 + len(ks)], want)
    assert q[0, 0] == 127 and q[1, 0] == -127


def test_all_codes_reachable(orc):
    x = np.zeros((1, 256), dtype=np.float32)
    x[0, :255] = np.arange(-127, 128) * 2.0 ** -7
    _, q, _ = q8K_fields(orc.quantize_q8K(x))
    assert np.array_equal(q[0, :255], np.arange(-127, 128))


def test_odd_symmetry_and_pow2_invariance(orc):
    rng = np.random.default_rng(2)
    x = _rand(rng, 5, 768)
    d0, q0, s0 = q8K_fields(orc.quantize_q8K(x))
    d1, q1, s1 = q8K_fields(orc.quantize_q8K(-x))
    assert np.array_equal(q1, -q0) and np.array_equal(s1, -s0) and np.array_equal(d1, d0)
    for p in (-3, 5):
        d2, q2, _ = q8K_fields(orc.quantize_q8K(x * np.float32(2.0 ** p)))
        assert np.array_equal(q2, q0)
        assert np.array_equal(d2, d0 * np.float32(2.0 ** p))


def test_zero_block_and_tiny_values(orc):
    x = np.zeros((2, 512), dtype=np.float32)
    x[1, 256:] = np.float32(1e-40)  # subnormal block, amax/127 underflows towards 0
    x[1, 300] = np.float32(-3e-39)
    xq = orc.quantize_q8K(x)
    d, q, s = q8K_fields(xq)
    assert np.all(d[:3] == 0) and np.all(q[:3] == 0) and np.all(s[:3] == 0)
    assert d[3] > 0 and q[3].min() == -127


def test_rows_independent(orc):
    # a block's bytes depend only on its own 256 values
    rng = np.random.default_rng(9)
    x = _rand(rng, 6, 512)
    full = orc.quantize_q8K(x)
    for m in range(6):
        assert np.array_equal(orc.quantize_q8K(x[m:m + 1]), full[m:m + 1])
