"""GPU: the four-tile q4_K GEMM (launches of 1024 activation rows and more, and
of 576..1023 where the grid favours it) against the oracle and against the
two-tile kernel.

The two kernels form the same int32 sums (sc = 8a + b folded into two int8
planes, combined as 8A + B), the same f16 min term and the same f32 epilogue in
the same order, and split a row over two K-groups by K alone (32 super-blocks
or more), so a launch's choice between them changes no bits: every output of a
large call equals the same row in a call of fewer than 1024 rows, bit for bit.
The shapes take the paths of the activation loads (17 16-byte loads per 32
rows, the last ones by two waves only): a ragged last row tile (rows past M
read as zero), column tails (N not a multiple of 128), rows of one super-block,
the K split with an even and an odd super-block count (the second group's idle
last step), and the SiLU form on an odd number of outputs.  The oracle checks
sampled rows (first and last included) within 1e-5 * sum_k|w_k * xhat_k| + 1e-6,
and exactly in the exact-integer regime.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from quant_packed_weight_amd import synth
from test_gpu_exact import LIMIT, assert_bits, exact_weights, q8K_bytes

pytestmark = pytest.mark.gpu

Q4 = 12


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def _rows(M, n=16, seed=5):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, M - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], mid])).astype(np.int64)


# (N, K, M): ragged rows and columns; one super-block; the K split on 32 (even)
# and 49 (odd) super-blocks; a full gate/up-sized launch; a q/k/v-sized launch
# below 1024 rows that the grid rule gives the four-tile kernel (its 600-row
# subset takes the two-tile kernel)
@pytest.mark.parametrize("N,K,M", [(1000, 256, 1100), (130, 8192, 1024), (300, 12544, 1030),
                                   (24576, 4096, 1024), (6144, 4096, 700)])
def test_four_tile_equals_two_tile(dev, gq, orc, N, K, M):
    log("q4_K four-tile N=%d K=%d M=%d" % (N, K, M))
    rng = np.random.default_rng(N + K + M)
    W = synth.make_weights(rng, Q4, N, K)
    x = synth.make_activations(rng, M, K, True)
    xq = orc.quantize_q8K(x)
    Wd, xqd = to_dev(W), to_dev(xq)
    full = to_host(gq.gemm(Q4, Wd, xqd, M, N, K, path=gq.PATH_GEMM))
    for a, b in [(0, 3), (M - 5, M), (M // 2, M // 2 + 77), (M - 600, M)]:
        part = to_host(gq.gemm(Q4, Wd, to_dev(xq[a:b]), b - a, N, K, path=gq.PATH_GEMM))
        assert np.array_equal(part.view(np.uint32), full[a:b].view(np.uint32)), (a, b)
    rows = _rows(M)
    yo = orc.gemm_int(Q4, W, xq, M, N, K, rows)
    _, S = orc.gemm_dequant(Q4, W, xq, M, N, K, rows)
    assert_within(full[rows], yo, S, "q4_K four-tile")


@pytest.mark.parametrize("N,K", [(130, 4096), (70, 12544)])
def test_four_tile_exact(dev, gq, orc, N, K):
    # power-of-two scales and activations small enough that every partial sum is
    # exact in f32: the sampled rows equal the oracle bit for bit
    M = 1100
    log("q4_K four-tile exact N=%d K=%d" % (N, K))
    rng = np.random.default_rng(40 + K)
    W, mag = exact_weights(rng, Q4, N, K)
    nb = K // 256
    dx = 2.0 ** -rng.integers(7, 9, (M, nb))
    colmax = mag.max(0)
    qx = rng.integers(-2, 3, (M, K)) * (rng.random((M, K)) < 0.5)
    for m in range(M):
        while (colmax * np.repeat(dx[m], 256) * np.abs(qx[m])).sum() > LIMIT:
            nz = np.flatnonzero(qx[m])
            qx[m, rng.choice(nz, (nz.size + 1) // 2, replace=False)] = 0
    xq = q8K_bytes(dx, qx)
    got = to_host(gq.gemm(Q4, to_dev(W), to_dev(xq), M, N, K, path=gq.PATH_GEMM))
    rows = _rows(M, 32)
    want = orc.gemm_int(Q4, W, xq, M, N, K, rows)
    w32 = want.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), want), "case leaves the exact regime"
    assert_bits(got[rows], w32, "q4_K four-tile exact K %d" % K)


def test_four_tile_silu(dev, gq):
    # gate/up with the SiLU product on the four-tile kernel: equal bit for bit to
    # a three-row call (two-tile kernel), and silu(G) * U of the group call's own
    # G, U within the product's f32 roundings; 1000 outputs leave a ragged pair
    # tile
    N, K, M = 1000, 4096, 1100
    log("q4_K four-tile silu")
    rng = np.random.default_rng(56)
    x = synth.make_activations(rng, M, K, True)
    xd = to_dev(x)
    wg = to_dev(synth.make_weights(rng, Q4, N, K))
    wu = to_dev(synth.make_weights(rng, Q4, N, K))
    y, xq = gq.linear_silu_mul(Q4, wg, wu, xd, N, path=gq.PATH_GEMM)
    y = to_host(y)
    for a in (0, 517, M - 3):
        ys, _ = gq.linear_silu_mul(Q4, wg, wu, to_dev(x[a:a + 3]), N, path=gq.PATH_GEMM)
        assert np.array_equal(to_host(ys).view(np.uint32), y[a:a + 3].view(np.uint32)), a
    G, U = gq.gemm_group(Q4, [wg, wu], xq, M, [N, N], K, path=gq.PATH_GEMM)
    g = to_host(G).astype(np.float64)
    u = to_host(U).astype(np.float64)
    yd = g / (1.0 + np.exp(-np.clip(g, -700, 700))) * u
    err = np.abs(y.astype(np.float64) - yd)
    assert (err <= 8 * 2.0 ** -24 * np.abs(yd) + np.abs(g * u) * 2.0 ** -126 + 2.0 ** -149).all()
