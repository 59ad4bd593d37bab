"""GPU: the small-M q4_K MFMA kernel (GEMMQ_PATH_SKINNY, batched decode) against
the CPU oracle, element by element within 1e-5 * sum_k|w_k * xhat_k| + 1e-6.

Bit identity inside the path: the split of a row's super-blocks over the waves
depends on K only and MFMA rows are independent, so an output does not depend on
M or on which other rows are in the call -- also across the forms with one to
four 16-row tiles (M <= 16, 32, 48, 64).  Shapes cover row lengths that give
one to eight waves per workgroup and several super-blocks per wave, N tails
(columns past N in a 16-column tile), M past 4-row output groups, and blocks
with extreme scales and values.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from quant_packed_weight_amd import synth

pytestmark = pytest.mark.gpu

Q4 = 12


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def _case(orc, M, N, K, seed):
    rng = np.random.default_rng(seed)
    W = synth.make_weights(rng, Q4, N, K)
    x = synth.make_activations(rng, M, K, True)
    return W, x, orc.quantize_q8K(x)


def _check(gq, orc, W, xq, M, N, K, where):
    y = to_host(gq.gemm(Q4, to_dev(W), to_dev(xq), M, N, K, path=gq.PATH_SKINNY))
    yo = orc.gemm_int(Q4, W, xq, M, N, K)
    _, S = orc.gemm_dequant(Q4, W, xq, M, N, K)
    assert_within(y, yo, S, where)
    return y


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 11, 16, 17, 24, 32, 33, 40, 48, 49, 64])
@pytest.mark.parametrize("N,K", [(1, 256), (15, 512), (17, 768), (100, 1024), (33, 2304),
                                 (40, 4096), (16, 8192), (21, 12288), (7, 20480)])
def test_skinny_parity(dev, gq, orc, M, N, K):
    log("skinny M=%d N=%d K=%d" % (M, N, K))
    W, _, xq = _case(orc, M, N, K, seed=13 * M + 7 * N + K)
    _check(gq, orc, W, xq, M, N, K, "skinny")


@pytest.mark.parametrize("K", [1024, 4608, 12288])
def test_skinny_rows_independent_of_call(dev, gq, orc, K):
    log("skinny row-subset K=%d" % K)
    M, N = 64, 70
    W, _, xq = _case(orc, M, N, K, seed=K + 1)
    Wd = to_dev(W)
    full = _check(gq, orc, W, xq, M, N, K, "skinny full")
    for a, b in [(0, 1), (3, 4), (0, 8), (5, 16), (15, 16), (2, 13), (0, 17), (16, 32),
                 (7, 31), (31, 32), (0, 33), (10, 50), (40, 64), (63, 64), (1, 49)]:
        part = to_host(gq.gemm(Q4, Wd, to_dev(xq[a:b]), b - a, N, K, path=gq.PATH_SKINNY))
        assert np.array_equal(part.view(np.uint32), full[a:b].view(np.uint32)), (a, b)


@pytest.mark.parametrize("M", [32, 64])
def test_skinny_extreme_blocks(dev, gq, orc, M):
    # every scale and min at 63, quants at 0 or 15, f16 d / dmin at large, tiny
    # and negative values, activations at +-amax
    log("skinny extreme blocks M=%d" % M)
    rng = np.random.default_rng(99)
    N, K = 48, 2048
    nb = K // 256
    W = synth.make_weights(rng, Q4, N, K).reshape(N * nb, 144).copy()
    d = np.array([65504.0, 6.0e-8, -3.5, 1.0], dtype=np.float16)
    for i in range(N * nb):
        W[i, 0:2] = d[rng.integers(0, 4, 1)].view(np.uint8)
        W[i, 2:4] = d[rng.integers(0, 4, 1)].view(np.uint8)
        if i % 3 == 0:
            W[i, 4:16] = 0xFF  # every 6-bit scale and min at 63
        if i % 5 == 0:
            W[i, 16:] = rng.choice(np.array([0x00, 0xFF, 0x0F, 0xF0], dtype=np.uint8), 128)
    W = W.reshape(N, -1)
    x = synth.make_activations(rng, M, K, True)
    x[:, 0] = np.abs(x).max() * 3
    x[0, 1] = -x[0, 0]
    xq = orc.quantize_q8K(x)
    _check(gq, orc, W, xq, M, N, K, "skinny extreme")


@pytest.mark.parametrize("M", [3, 9, 16, 25, 41, 60])
def test_skinny_group_and_linear(dev, gq, orc, M):
    # a group launch (q/k/v-like) equals single calls; gemmq_linear_group takes
    # the same path automatically at these M and gives the same bits
    log("skinny group M=%d" % M)
    K = 4096
    Ns = [300, 64, 65]
    rng = np.random.default_rng(50 + M)
    Ws = [synth.make_weights(rng, Q4, N, K) for N in Ns]
    x = synth.make_activations(rng, M, K, True)
    xd = to_dev(x)
    Wd = [to_dev(W) for W in Ws]
    xq = gq.quantize_q8K(xd)
    outs = gq.gemm_group(Q4, Wd, xq, M, Ns, K, path=gq.PATH_SKINNY)
    for W, N, o in zip(Wd, Ns, outs):
        single = to_host(gq.gemm(Q4, W, xq, M, N, K, path=gq.PATH_SKINNY))
        assert np.array_equal(to_host(o).view(np.uint32), single.view(np.uint32)), N
    lin, xq2 = gq.linear_group(Q4, Wd, xd, Ns)
    assert np.array_equal(to_host(xq2), to_host(xq))
    for o, r in zip(lin, outs):
        assert np.array_equal(to_host(o).view(np.uint32), to_host(r).view(np.uint32))
    xq_o = orc.quantize_q8K(x)
    yo = orc.gemm_int(Q4, Ws[0], xq_o, M, Ns[0], K)
    _, S = orc.gemm_dequant(Q4, Ws[0], xq_o, M, Ns[0], K)
    assert_within(to_host(outs[0]), yo, S, "skinny group")


@pytest.mark.parametrize("M", [4, 8, 16, 32, 47, 64])
def test_skinny_silu_route(dev, gq, M):
    # gemmq_linear_silu_mul on this path: the automatic choice and the forced
    # path agree bit for bit, and equal silu(G) * U of this path's own G, U to
    # within the f32 roundings of the product (a swapped or misaligned pair
    # would miss by far)
    log("skinny silu M=%d" % M)
    rng = np.random.default_rng(600 + M)
    K, N = 3072, 77
    x = to_dev(synth.make_activations(rng, M, K, True))
    wg = to_dev(synth.make_weights(rng, Q4, N, K))
    wu = to_dev(synth.make_weights(rng, Q4, N, K))
    y, xq = gq.linear_silu_mul(Q4, wg, wu, x, N)
    y3, _ = gq.linear_silu_mul(Q4, wg, wu, x, N, path=gq.PATH_SKINNY)
    assert np.array_equal(to_host(y).view(np.uint32), to_host(y3).view(np.uint32))
    G, U = gq.gemm_group(Q4, [wg, wu], xq, M, [N, N], K, path=gq.PATH_SKINNY)
    g = to_host(G).astype(np.float64)
    u = to_host(U).astype(np.float64)
    yd = g / (1.0 + np.exp(-np.clip(g, -700, 700))) * u
    err = np.abs(to_host(y).astype(np.float64) - yd)
    assert (err <= 8 * 2.0 ** -24 * np.abs(yd) + np.abs(g * u) * 2.0 ** -126 + 2.0 ** -149).all()


def test_skinny_longest_rows(dev, gq, orc):
    # K at the library's limit (2^24, one row of 65536 super-blocks): eight waves
    # of 8192 super-blocks each, one to four row tiles
    K = 1 << 24
    for M, N in ((5, 3), (17, 2), (40, 1), (50, 1)):
        log("skinny longest rows M=%d N=%d" % (M, N))
        W, _, xq = _case(orc, M, N, K, seed=M + N)
        _check(gq, orc, W, xq, M, N, K, "skinny K=2^24")
