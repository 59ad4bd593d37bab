"""GPU: the load-time repack of q3_K and q6_K (gemmq_repack) and every route on
the repacked layouts.

The repacked bytes must equal the oracle's repack bit for bit.  The kernels
compute the same arithmetic in the same order whatever the layout, so on
repacked weights every output must equal the output on the original weights
bit for bit (GEMV at M = 1..8 over every launch shape, GEMM, grouped launches,
the fused layer, the SiLU pair), and one output per case is also checked
against the oracle within 1e-5 * sum_k|w_k * xhat_k| + 1e-6.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from quant_packed_weight_amd import synth

pytestmark = pytest.mark.gpu

Q3, Q6 = 11, 14
R = 256  # repacked = type id + 256


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def _same(a, b):
    return np.array_equal(to_host(a).view(np.uint32), to_host(b).view(np.uint32))


@pytest.mark.parametrize("fmt", [Q3, Q6])
@pytest.mark.parametrize("N,K", [(1, 256), (3, 768), (17, 4096), (1000, 1024), (7, 12288)])
def test_repack_bytes(dev, gq, orc, fmt, N, K):
    log("repack fmt=%d N=%d K=%d" % (fmt, N, K))
    W = synth.make_weights(np.random.default_rng(N + K + fmt), fmt, N, K)
    got = to_host(gq.repack(fmt, to_dev(W), N, K))
    assert np.array_equal(got.reshape(-1), orc.repack(fmt, W, N, K).reshape(-1))


@pytest.mark.parametrize("fmt", [Q3, Q6])
@pytest.mark.parametrize("M", [1, 2, 4, 5, 8])
@pytest.mark.parametrize("N,K", [(1, 256), (31, 512), (33, 1024), (1000, 2048), (130, 4096),
                                 (40, 8192), (33, 12288), (17, 20480)])
def test_gemv_same_bits(dev, gq, orc, fmt, M, N, K):
    log("gemv repacked fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    rng = np.random.default_rng(100 * M + N + K + fmt)
    W = synth.make_weights(rng, fmt, N, K)
    xq = orc.quantize_q8K(synth.make_activations(rng, M, K, True))
    Wd, xqd = to_dev(W), to_dev(xq)
    y = gq.gemm(fmt, Wd, xqd, M, N, K, path=gq.PATH_GEMV)
    yr = gq.gemm(fmt + R, gq.repack(fmt, Wd, N, K), xqd, M, N, K, path=gq.PATH_GEMV)
    assert _same(y, yr)
    if M in (1, 8):
        yo = orc.gemm_int(fmt, W, xq, M, N, K)
        _, S = orc.gemm_dequant(fmt, W, xq, M, N, K)
        assert_within(to_host(yr), yo, S, "gemv repacked")


@pytest.mark.parametrize("fmt", [Q3, Q6])
@pytest.mark.parametrize("M,N,K", [(9, 1, 256), (33, 200, 1024), (129, 127, 256), (300, 130, 3072),
                                   (40, 70, 8192), (600, 1500, 256)])
def test_gemm_same_bits(dev, gq, orc, fmt, M, N, K):
    log("gemm repacked fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    rng = np.random.default_rng(7 * M + 3 * N + K + fmt)
    W = synth.make_weights(rng, fmt, N, K)
    xq = orc.quantize_q8K(synth.make_activations(rng, M, K, True))
    Wd, xqd = to_dev(W), to_dev(xq)
    y = gq.gemm(fmt, Wd, xqd, M, N, K, path=gq.PATH_GEMM)
    yr = gq.gemm(fmt + R, gq.repack(fmt, Wd, N, K), xqd, M, N, K, path=gq.PATH_GEMM)
    assert _same(y, yr)
    yo = orc.gemm_int(fmt, W, xq, M, N, K)
    _, S = orc.gemm_dequant(fmt, W, xq, M, N, K)
    assert_within(to_host(yr), yo, S, "gemm repacked")


@pytest.mark.parametrize("fmt", [Q3, Q6])
@pytest.mark.parametrize("M,K,path", [(1, 1024, 0), (3, 4096, 0), (1, 12288, 0), (40, 1024, 0),
                                      (2, 2048, 2)])
def test_group_linear_and_silu_same_bits(dev, gq, orc, fmt, M, K, path):
    # a group of repacked matrices, the fused layer and the SiLU pair on repacked
    # weights give the bits of the same calls on the original weights
    log("group/linear/silu repacked fmt=%d M=%d K=%d path=%d" % (fmt, M, K, path))
    rng = np.random.default_rng(31 * M + K + fmt + path)
    Ns = [300, 65, 300]
    Ws = [to_dev(synth.make_weights(rng, fmt, N, K)) for N in Ns]
    Wr = [gq.repack(fmt, w, N, K) for w, N in zip(Ws, Ns)]
    x = to_dev(synth.make_activations(rng, M, K, True))
    xq = gq.quantize_q8K(x)
    for a, b in zip(gq.gemm_group(fmt, Ws, xq, M, Ns, K, path=path),
                    gq.gemm_group(fmt + R, Wr, xq, M, Ns, K, path=path)):
        assert _same(a, b)
    (la, qa), (lb, qb) = (gq.linear_group(fmt, Ws, x, Ns, path=path),
                          gq.linear_group(fmt + R, Wr, x, Ns, path=path))
    assert np.array_equal(to_host(qa), to_host(qb))
    for a, b in zip(la, lb):
        assert _same(a, b)
    sa, _ = gq.linear_silu_mul(fmt, Ws[0], Ws[2], x, 300, path=path)
    sb, _ = gq.linear_silu_mul(fmt + R, Wr[0], Wr[2], x, 300, path=path)
    assert _same(sa, sb)
