"""GPU: the small-M q6_K MFMA kernel (GEMMQ_PATH_SKINNY for q6_K and its
repacked layout, batched decode) against the CPU oracle, element by element
within 1e-5 * sum_k|w_k * xhat_k| + 1e-6.

Bit identity inside the path: the split of a row's super-blocks over the waves
depends on K only and MFMA rows are independent, so an output does not depend
on M or on which other rows are in the call -- also across the forms for
M <= 8 and M <= 16 -- and the repacked layout gives the original layout's bits.
Shapes cover row lengths that give one to eight waves per workgroup and several
super-blocks per wave, N tails (columns past N in a 32-column tile), M past
4-row output groups, and blocks with extreme scales, quants and factors.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from quant_packed_weight_amd import synth

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


def _case(orc, M, N, K, seed):
    rng = np.random.default_rng(seed)
    W = synth.make_weights(rng, Q6, N, K)
    x = synth.make_activations(rng, M, K, True)
    return W, x, orc.quantize_q8K(x)


def _run(gq, fmt, W, xq, M, N, K):
    w = to_dev(W)
    if fmt == Q6R:
        w = gq.repack(Q6, w, N, K)
    return to_host(gq.gemm(fmt, w, to_dev(xq), M, N, K, path=gq.PATH_SKINNY))


def _check(gq, orc, fmt, W, xq, M, N, K, where):
    y = _run(gq, fmt, W, xq, M, N, K)
    yo = orc.gemm_int(Q6, W, xq, M, N, K)
    _, S = orc.gemm_dequant(Q6, W, xq, M, N, K)
    assert_within(y, yo, S, where)
    return y


@pytest.mark.parametrize("fmt", [Q6, Q6R])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8, 9, 12, 13, 16])
@pytest.mark.parametrize("N,K", [(1, 256), (31, 512), (33, 768), (100, 1024), (64, 2304),
                                 (40, 4096), (17, 8192), (70, 12288), (5, 20480)])
def test_skinny_q6k_parity(dev, gq, orc, fmt, M, N, K):
    log("skinny q6_K fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    W, _, xq = _case(orc, M, N, K, seed=17 * M + 7 * N + K)
    _check(gq, orc, fmt, W, xq, M, N, K, "skinny q6_K")


@pytest.mark.parametrize("K", [1024, 4608, 12288])
def test_skinny_q6k_rows_independent_of_call(dev, gq, orc, K):
    log("skinny q6_K row-subset K=%d" % K)
    M, N = 16, 70
    W, _, xq = _case(orc, M, N, K, seed=K + 3)
    Wd = to_dev(W)
    full = _check(gq, orc, Q6, W, xq, M, N, K, "skinny q6_K full")
    rep = _run(gq, Q6R, W, xq, M, N, K)
    assert np.array_equal(rep.view(np.uint32), full.view(np.uint32))
    for a, b in [(0, 1), (3, 4), (0, 8), (5, 16), (15, 16), (2, 13), (8, 16), (7, 9), (0, 3)]:
        part = to_host(gq.gemm(Q6, Wd, to_dev(xq[a:b]), b - a, N, K, path=gq.PATH_SKINNY))
        assert np.array_equal(part.view(np.uint32), full[a:b].view(np.uint32)), (a, b)


@pytest.mark.parametrize("fmt", [Q6, Q6R])
@pytest.mark.parametrize("M", [8, 16])
@pytest.mark.parametrize("K", [2048, 4096])
def test_skinny_q6k_extreme_blocks(dev, gq, orc, fmt, M, K):
    # scales at -128 and 127, quants at 0 and 63, f16 d at large, tiny,
    # subnormal and negative values, activations at +-amax; K = 4096 takes the
    # plain layout's staged loads (blocks at both 4-byte phases)
    log("skinny q6_K extreme blocks fmt=%d M=%d K=%d" % (fmt, M, K))
    rng = np.random.default_rng(77)
    N = 48
    nb = K // 256
    W = synth.make_weights(rng, Q6, N, K).reshape(N * nb, 210).copy()
    d = np.array([65504.0, 6.0e-8, -3.5, 1.0, 2.0 ** -20], dtype=np.float16)
    for i in range(N * nb):
        W[i, 208:210] = d[rng.integers(0, 5, 1)].view(np.uint8)
        if i % 3 == 0:
            W[i, 192:208] = rng.choice(np.array([0x80, 0x7F], dtype=np.uint8), 16)
        if i % 4 == 0:
            W[i, 0:192] = rng.choice(np.array([0x00, 0xFF], dtype=np.uint8), 192)
    W = W.reshape(N, -1)
    x = synth.make_activations(rng, M, K, True)
    x[:, 0] = np.abs(x).max() * 3
    x[0, 1] = -x[0, 0]
    xq = orc.quantize_q8K(x)
    _check(gq, orc, fmt, W, xq, M, N, K, "skinny q6_K extreme")


@pytest.mark.parametrize("M", [3, 8, 11, 16])
@pytest.mark.parametrize("K", [2048, 4096])
def test_skinny_q6k_group_and_linear(dev, gq, orc, M, K):
    # a group launch equals single calls; gemmq_linear_group on this path
    # gives the same bits (and so does its automatic choice at M > 8, and at
    # 5 <= M <= 8 past 16384 columns -- checked in the dispatch tests)
    # (K = 4096: the plain layout's staged loads)
    log("skinny q6_K group M=%d K=%d" % (M, K))
    Ns = [300, 64, 65]
    rng = np.random.default_rng(80 + M)
    Ws = [synth.make_weights(rng, Q6, N, K) for N in Ns]
    x = synth.make_activations(rng, M, K, True)
    xd = to_dev(x)
    Wd = [to_dev(W) for W in Ws]
    xq = gq.quantize_q8K(xd)
    outs = gq.gemm_group(Q6, Wd, xq, M, Ns, K, path=gq.PATH_SKINNY)
    for W, N, o in zip(Wd, Ns, outs):
        single = to_host(gq.gemm(Q6, W, xq, M, N, K, path=gq.PATH_SKINNY))
        assert np.array_equal(to_host(o).view(np.uint32), single.view(np.uint32)), N
    lin, xq2 = gq.linear_group(Q6, Wd, xd, Ns, path=gq.PATH_SKINNY)
    assert np.array_equal(to_host(xq2), to_host(xq))
    if M > 8:
        auto, _ = gq.linear_group(Q6, Wd, xd, Ns)
        for o, r in zip(auto, outs):
            assert np.array_equal(to_host(o).view(np.uint32), to_host(r).view(np.uint32))
    for o, r in zip(lin, outs):
        assert np.array_equal(to_host(o).view(np.uint32), to_host(r).view(np.uint32))
    xq_o = orc.quantize_q8K(x)
    for W, N, o in zip(Ws, Ns, outs):
        yo = orc.gemm_int(Q6, W, xq_o, M, N, K)
        _, S = orc.gemm_dequant(Q6, W, xq_o, M, N, K)
        assert_within(to_host(o), yo, S, "skinny q6_K group")


@pytest.mark.parametrize("M", [4, 8, 16])
def test_skinny_q6k_silu_route(dev, gq, M):
    # gemmq_linear_silu_mul on this path (at M > 8 also the automatic choice,
    # bit for bit) equals silu(G) * U of this path's own G, U to
    # within the f32 roundings of the product (a swapped or misaligned pair
    # would miss by far)
    log("skinny q6_K silu M=%d" % M)
    rng = np.random.default_rng(700 + M)
    K, N = 3072, 77
    x = to_dev(synth.make_activations(rng, M, K, True))
    wg = to_dev(synth.make_weights(rng, Q6, N, K))
    wu = to_dev(synth.make_weights(rng, Q6, N, K))
    y, xq = gq.linear_silu_mul(Q6, wg, wu, x, N, path=gq.PATH_SKINNY)
    if M > 8:  # the automatic choice at these M (fewer than 16384 columns)
        y3, _ = gq.linear_silu_mul(Q6, wg, wu, x, N)
        assert np.array_equal(to_host(y).view(np.uint32), to_host(y3).view(np.uint32))
    G, U = gq.gemm_group(Q6, [wg, wu], xq, M, [N, N], K, path=gq.PATH_SKINNY)
    g = to_host(G).astype(np.float64)
    u = to_host(U).astype(np.float64)
    yd = g / (1.0 + np.exp(-np.clip(g, -700, 700))) * u
    err = np.abs(to_host(y).astype(np.float64) - yd)
    assert (err <= 8 * 2.0 ** -24 * np.abs(yd) + np.abs(g * u) * 2.0 ** -126 + 2.0 ** -149).all()


def test_skinny_q6k_longest_rows(dev, gq, orc):
    # K at the library's limit (2^24, one row of 65536 super-blocks): eight waves
    # of 8192 super-blocks each
    K = 1 << 24
    for M, N in ((5, 3), (16, 2)):
        log("skinny q6_K longest rows M=%d N=%d" % (M, N))
        W, _, xq = _case(orc, M, N, K, seed=M + N)
        _check(gq, orc, Q6, W, xq, M, N, K, "skinny q6_K K=2^24")
