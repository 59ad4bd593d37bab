"""GPU: the four-tile q6_K GEMM (taken on grids of 2048 workgroups and more)
against the oracle and against the plane kernel.

The two kernels form the same exact integer sum per super-block and output
(sum_j sc_j (q - 32) . x in int32) and the same f32 epilogue in the same
order, so a launch's choice between them changes no bits: every output of a
large call equals the same row in a small call (which the plane kernel runs),
bit for bit.  Shapes: short rows (one and two super-blocks), long rows (32
super-blocks), the plain and the repacked layout, the SiLU-gated form; the
oracle checks sampled rows (first and last included) within
1e-5 * sum_k|w_k * xhat_k| + 1e-6, and exactly in the exact-integer regime.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from quant_packed_weight_amd import synth
from test_gpu_exact import LIMIT, assert_bits, exact_weights, q8K_bytes

pytestmark = pytest.mark.gpu

Q6 = 14
Q6R = 256 + 14


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def _rows(M, n=16, seed=7):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, M - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], mid])).astype(np.int64)


def _weights_dev(gq, fmt, W, N, K):
    w = to_dev(W)
    return gq.repack(Q6, w, N, K) if fmt == Q6R else w


# grids: 128 x 16, 512 x 4, 128 x 16 workgroups of 128 x 128
@pytest.mark.parametrize("fmt", [Q6, Q6R])
@pytest.mark.parametrize("N,K,M", [(16384, 256, 2048), (65536, 512, 512), (16384, 8192, 2048)])
def test_four_tile_equals_plane_kernel(dev, gq, orc, fmt, N, K, M):
    log("q6_K four-tile fmt=%d N=%d K=%d M=%d" % (fmt, N, K, M))
    rng = np.random.default_rng(N + K + M + fmt)
    W = synth.make_weights(rng, Q6, N, K)
    x = synth.make_activations(rng, M, K, True)
    xq = orc.quantize_q8K(x)
    Wd, xqd = _weights_dev(gq, fmt, W, N, K), to_dev(xq)
    full = to_host(gq.gemm(fmt, Wd, xqd, M, N, K, path=gq.PATH_GEMM))
    for a, b in [(0, 3), (M - 5, M), (M // 2, M // 2 + 17)]:
        part = to_host(gq.gemm(fmt, Wd, to_dev(xq[a:b]), b - a, N, K, path=gq.PATH_GEMM))
        assert np.array_equal(part.view(np.uint32), full[a:b].view(np.uint32)), (a, b)
    rows = _rows(M)
    yo = orc.gemm_int(Q6, W, xq, M, N, K, rows)
    _, S = orc.gemm_dequant(Q6, W, xq, M, N, K, rows)
    assert_within(full[rows], yo, S, "q6_K four-tile")


@pytest.mark.parametrize("fmt", [Q6, Q6R])
def test_four_tile_exact(dev, gq, orc, fmt):
    # power-of-two scales and activations small enough that every partial sum
    # is exact in f32: the sampled rows equal the oracle bit for bit
    N, K, M = 16384, 256, 2048
    log("q6_K four-tile exact fmt=%d" % fmt)
    rng = np.random.default_rng(90 + fmt)
    W, mag = exact_weights(rng, Q6, N, K)
    nb = K // 256
    dx = 2.0 ** -rng.integers(7, 9, (M, nb))
    # bound every output by the column maxima of the weight magnitudes
    colmax = mag.max(0)
    qx = rng.integers(-2, 3, (M, K)) * (rng.random((M, K)) < 0.5)
    for m in range(M):
        while (colmax * np.repeat(dx[m], 256) * np.abs(qx[m])).sum() > LIMIT:
            nz = np.flatnonzero(qx[m])
            qx[m, rng.choice(nz, (nz.size + 1) // 2, replace=False)] = 0
    xq = q8K_bytes(dx, qx)
    got = to_host(gq.gemm(fmt, _weights_dev(gq, fmt, W, N, K), to_dev(xq), M, N, K))
    rows = _rows(M, 32)
    want = orc.gemm_int(Q6, W, xq, M, N, K, rows)
    w32 = want.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), want), "case leaves the exact regime"
    assert_bits(got[rows], w32, "q6_K four-tile exact fmt %d" % fmt)


def test_four_tile_silu(dev, gq):
    # gate/up in q6_K with the SiLU product on the GEMM path: the large call
    # (four-tile kernel) equals a three-row call (plane kernel) bit for bit,
    # and silu(G) * U of the group call's own G, U within the product's f32
    # roundings
    N, K, M = 16384, 512, 1024
    log("q6_K four-tile silu")
    rng = np.random.default_rng(55)
    x = synth.make_activations(rng, M, K, True)
    xd = to_dev(x)
    wg = to_dev(synth.make_weights(rng, Q6, N, K))
    wu = to_dev(synth.make_weights(rng, Q6, N, K))
    y, xq = gq.linear_silu_mul(Q6, wg, wu, xd, N, path=gq.PATH_GEMM)
    y = to_host(y)
    ys, _ = gq.linear_silu_mul(Q6, wg, wu, to_dev(x[100:103]), N, path=gq.PATH_GEMM)
    assert np.array_equal(to_host(ys).view(np.uint32), y[100:103].view(np.uint32))
    G, U = gq.gemm_group(Q6, [wg, wu], xq, M, [N, N], K, path=gq.PATH_GEMM)
    g = to_host(G).astype(np.float64)
    u = to_host(U).astype(np.float64)
    yd = g / (1.0 + np.exp(-np.clip(g, -700, 700))) * u
    err = np.abs(y.astype(np.float64) - yd)
    assert (err <= 8 * 2.0 ** -24 * np.abs(yd) + np.abs(g * u) * 2.0 ** -126 + 2.0 ** -149).all()
