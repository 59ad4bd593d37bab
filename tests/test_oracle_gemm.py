"""Pins of the oracle's packed matmul (CPU only).

Checks: exact rational sums on tiny cases built by the independent packer; a
reduction to a textbook integer GEMM (numpy int64 matmul) with no tolerance; the
two oracle routes (integer decomposition, decode-then-dot) against each other at
the bound the f32 decode rounding allows; row-subset equality (the pages' tiled
equals single-row rule, molayo article, status row "src/ -- C++ engine"); and
exact power-of-two linearity.
"""
from fractions import Fraction

import numpy as np
import pytest

from packer import pack_q4K, pack_q6K, q8K_fields
from quant_packed_weight_amd import synth

Q4, Q6 = 12, 14


def _fields_q4K(rng, n):
    d = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    dmin = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    return d, dmin, rng.integers(0, 64, (n, 8)), rng.integers(0, 64, (n, 8)), rng.integers(0, 16, (n, 256))


def _fields_q6K(rng, n):
    d = (np.abs(rng.standard_normal(n)) * 1e-3).astype(np.float16)
    return d, rng.integers(-128, 128, (n, 16)), rng.integers(0, 64, (n, 256))


@pytest.mark.parametrize("fmt", [Q4, Q6])
def test_exact_rational_tiny(orc, fmt):
    # y = sum_k w_k * xhat_k with the unrounded w_k built from the packer's fields
    rng = np.random.default_rng(21 + fmt)
    N, K, M = 3, 512, 2
    nb = K // 256
    if fmt == Q4:
        d, dmin, sc, mn, q = _fields_q4K(rng, N * nb)
        W = pack_q4K(d, dmin, sc, mn, q).reshape(N, -1)
    else:
        d, sc, q = _fields_q6K(rng, N * nb)
        W = pack_q6K(d, sc, q).reshape(N, -1)
    x = rng.standard_normal((M, K)).astype(np.float32)
    xq = orc.quantize_q8K(x)
    dx, qx, _ = q8K_fields(xq)
    ya = orc.gemm_int(fmt, W, xq, M, N, K)
    yb, S = orc.gemm_dequant(fmt, W, xq, M, N, K)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            for b in range(nb):
                blk = n * nb + b
                fdx = Fraction(float(dx[m * nb + b]))
                for i in range(256):
                    if fmt == Q4:
                        j = i // 32
                        w = (Fraction(float(d[blk])) * int(sc[blk, j]) * int(q[blk, i])
                             - Fraction(float(dmin[blk])) * int(mn[blk, j]))
                    else:
                        w = Fraction(float(d[blk])) * int(sc[blk, i // 16]) * (int(q[blk, i]) - 32)
                    exact += w * fdx * int(qx[m * nb + b, i])
            s = S[m, n]
            assert abs(Fraction(float(ya[m, n])) - exact) <= Fraction(1e-15) * Fraction(s)
            # the decode-then-dot route rounds each q4_K weight once to f32
            bound = (2.0 ** -24 if fmt == Q4 else 0.0) * s + 1e-15 * s
            assert abs(Fraction(float(yb[m, n])) - exact) <= Fraction(bound)


@pytest.mark.parametrize("fmt", [Q4, Q6])
def test_textbook_integer_gemm(orc, fmt):
    # scales 1, mins 0, d_w = 2^-10 and activations with d_x = 2^-7 exactly:
    # y = 2^-17 * (integer matmul), with no tolerance at all.
    rng = np.random.default_rng(31 + fmt)
    N, K, M = 17, 768, 5
    nb = K // 256
    if fmt == Q4:
        qw = rng.integers(0, 16, (N * nb, 256))
        W = pack_q4K(np.full(N * nb, 2.0 ** -10), np.zeros(N * nb), np.ones((N * nb, 8), int),
                     np.zeros((N * nb, 8), int), qw).reshape(N, -1)
        wint = qw.reshape(N, K)
    else:
        qw = rng.integers(0, 64, (N * nb, 256))
        W = pack_q6K(np.full(N * nb, 2.0 ** -10), np.ones((N * nb, 16), int), qw).reshape(N, -1)
        wint = qw.reshape(N, K) - 32
    k = rng.integers(-127, 128, (M, K))
    k[:, ::256] = 127  # every block has amax = 127 * 2^-7, so d_x = 2^-7 and q_x = k
    x = (k * 2.0 ** -7).astype(np.float32)
    xq = orc.quantize_q8K(x)
    dx, qx, _ = q8K_fields(xq)
    assert np.all(dx == np.float32(2.0 ** -7)) and np.array_equal(qx.reshape(M, K), k)
    want = (k.astype(np.int64) @ wint.T.astype(np.int64)) * 2.0 ** -17
    assert np.array_equal(orc.gemm_int(fmt, W, xq, M, N, K), want)
    yb, _ = orc.gemm_dequant(fmt, W, xq, M, N, K)
    assert np.array_equal(yb, want)


@pytest.mark.parametrize("fmt", [Q4, Q6])
def test_routes_agree(orc, fmt):
    rng = np.random.default_rng(41 + fmt)
    N, K, M = 64, 2048, 9
    W = synth.make_weights(rng, fmt, N, K)
    xq = orc.quantize_q8K(synth.make_activations(rng, M, K, True))
    ya = orc.gemm_int(fmt, W, xq, M, N, K)
    yb, S = orc.gemm_dequant(fmt, W, xq, M, N, K)
    bound = (2.0 ** -23 if fmt == Q4 else 1e-13) * S
    assert np.all(np.abs(ya - yb) <= bound)
    assert np.all(S > 0)


@pytest.mark.parametrize("fmt", [Q4, Q6])
def test_row_subset_bit_identical(orc, fmt):
    rng = np.random.default_rng(51 + fmt)
    N, K, M = 40, 512, 11
    W = synth.make_weights(rng, fmt, N, K)
    xq = orc.quantize_q8K(synth.make_activations(rng, M, K, True))
    full = orc.gemm_int(fmt, W, xq, M, N, K)
    fullb, fullS = orc.gemm_dequant(fmt, W, xq, M, N, K)
    rows = np.array([10, 0, 7, 7, 3])
    assert np.array_equal(orc.gemm_int(fmt, W, xq, M, N, K, rows=rows), full[rows])
    yb, S = orc.gemm_dequant(fmt, W, xq, M, N, K, rows=rows)
    assert np.array_equal(yb, fullb[rows]) and np.array_equal(S, fullS[rows])
    for m in range(M):
        one = orc.gemm_int(fmt, W, xq[m:m + 1], 1, N, K)
        assert np.array_equal(one[0], full[m])


@pytest.mark.parametrize("fmt", [Q4, Q6])
def test_power_of_two_linearity(orc, fmt):
    rng = np.random.default_rng(61 + fmt)
    N, K, M = 16, 512, 3
    W = synth.make_weights(rng, fmt, N, K)
    x = synth.make_activations(rng, M, K, True)
    xq = orc.quantize_q8K(x)
    y = orc.gemm_int(fmt, W, xq, M, N, K)
    # doubling every f16 scale field doubles y exactly
    W2 = W.copy().reshape(-1, 144 if fmt == Q4 else 210)
    offs = (0, 2) if fmt == Q4 else (208,)
    for o in offs:
        f = W2[:, o:o + 2].copy().view(np.float16) * np.float16(2)
        W2[:, o:o + 2] = f.view(np.uint8)
    y2 = orc.gemm_int(fmt, W2.reshape(N, -1), xq, M, N, K)
    assert np.array_equal(y2, 2 * y)
    # scaling the activations by 4 scales y by 4 exactly
    y4 = orc.gemm_int(fmt, W, orc.quantize_q8K(x * np.float32(4)), M, N, K)
    assert np.array_equal(y4, 4 * y)


def test_bad_args(orc):
    with pytest.raises(ValueError):
        orc.quantize_q8K(np.zeros((1, 300), np.float32))
    with pytest.raises(ValueError):
        orc.gemm_int(99, np.zeros((1, 144), np.uint8), np.zeros((1, 292), np.uint8), 1, 1, 256)
