"""GPU: the GEMV's staged form against the plain and the fused forms and the oracle.

Large decode launches (rows x M x blocks per row from 2^18) stage the q8_K
blocks in each workgroup's LDS instead of reading activation fragments from L2
per lane (the plain form); from f32 activations, launches from 2^19 (from 2^18
where each wave would quantize four blocks) run the quantizer on its own and
then the staged form instead of quantizing in every workgroup (the fused form).  All three forms give every output the same integer
sums and f32 steps in the same order, so they must agree bit for bit: a large
call's first rows against a call on those rows alone (small: plain or fused),
the one-call layer against quantize + gemm (the GEMV path forced: from M = 3 the
automatic choice may take the small-M kernel, whose bits differ).  Sampled
outputs are checked against the oracle within 1e-5 * sum_k|w_k * xhat_k| + 1e-6.
The shapes take each row
layout of the GEMV (16 / 8 / 4 blocks a row: one, two and four rows side by side
per wave) at M = 1, 2 and 4.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from quant_packed_weight_amd import synth

pytestmark = pytest.mark.gpu

Q2, Q3, Q4, Q5, Q6 = 10, 11, 12, 13, 14
R = 256
PATH_GEMV = 1
SUB = 1000  # rows of the small comparison call (below every threshold)


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def _weights(gq, fmt, W, N, K):
    w = to_dev(W)
    return gq.repack(fmt & 255, w, N, K) if fmt > 255 else w


def _cols(N, n=24, seed=3):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, N - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, N - 1], mid]))


def _check_oracle(orc, fmt, W, xq, M, N, K, got, where):
    # the oracle on a subset of the weight rows (output columns)
    cols = _cols(N)
    Ws = np.ascontiguousarray(W[cols])
    yo = orc.gemm_int(fmt & 255, Ws, xq, M, len(cols), K)
    _, S = orc.gemm_dequant(fmt & 255, Ws, xq, M, len(cols), K)
    assert_within(got[:, cols], yo, S, where)


# (M, K, N): rows x M x K/256 = 320000 (staged when the q8_K blocks are given,
# fused from f32 activations), and the staged form where the fused one does not
# reach: 64 blocks at M = 4, the 8-row form at M = 6 and 8 (the layer call then
# quantizes in a launch of its own)
@pytest.mark.parametrize("fmt", [Q4, Q6, Q2, Q3, Q5, R + Q6])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 20000), (2, 2048, 20000), (4, 1024, 20000),
                                   (4, 4096, 5000), (6, 2048, 20000), (8, 1024, 20000)])
def test_staged_equals_plain_and_fused(dev, gq, orc, fmt, M, K, N):
    log("gemv staged fmt=%d M=%d K=%d N=%d" % (fmt, M, K, N))
    rng = np.random.default_rng(fmt + 7 * M + K)
    W = synth.make_weights(rng, fmt & 255, N, K)
    x = synth.make_activations(rng, M, K, True)
    xq = orc.quantize_q8K(x)
    xqd = to_dev(xq)
    staged = to_host(gq.gemm(fmt, _weights(gq, fmt, W, N, K), xqd, M, N, K, path=PATH_GEMV))
    plain = to_host(gq.gemm(fmt, _weights(gq, fmt, W[:SUB], SUB, K), xqd, M, SUB, K, path=PATH_GEMV))
    assert np.array_equal(staged[:, :SUB].view(np.uint32), plain.view(np.uint32))
    fused, xq2 = gq.linear_group(fmt, [_weights(gq, fmt, W, N, K)], to_dev(x), [N], path=PATH_GEMV)
    assert np.array_equal(to_host(xq2), xq)
    assert np.array_equal(to_host(fused[0]).view(np.uint32), staged.view(np.uint32))
    _check_oracle(orc, fmt, W, xq, M, N, K, staged, "staged")


# rows x M x K/256 = 640000, and at M = 3, 4 with rows of 8 blocks (four blocks a
# wave to quantize) 294912 and 262400: the one-call layer quantizes in a launch
# of its own and runs the staged form; 262080 (M = 4) stays fused.  Equal to the
# fused form on a few of its rows either way
@pytest.mark.parametrize("fmt", [Q4, Q6, R + Q6])
@pytest.mark.parametrize("M,K,N", [(2, 4096, 20000), (1, 2048, 80000), (3, 2048, 12288),
                                   (4, 2048, 8200), (4, 2048, 8190)])
def test_layer_split_quantizer(dev, gq, orc, fmt, M, K, N):
    log("gemv layer split fmt=%d M=%d K=%d N=%d" % (fmt, M, K, N))
    rng = np.random.default_rng(100 + fmt + M + K)
    W = synth.make_weights(rng, fmt & 255, N, K)
    x = synth.make_activations(rng, M, K, True)
    xq = orc.quantize_q8K(x)
    xd = to_dev(x)
    big, xq2 = gq.linear_group(fmt, [_weights(gq, fmt, W, N, K)], xd, [N], path=PATH_GEMV)
    assert np.array_equal(to_host(xq2), xq)
    big = to_host(big[0])
    small, _ = gq.linear_group(fmt, [_weights(gq, fmt, W[:SUB], SUB, K)], xd, [SUB], path=PATH_GEMV)
    assert np.array_equal(big[:, :SUB].view(np.uint32), to_host(small[0]).view(np.uint32))
    _check_oracle(orc, fmt, W, xq, M, N, K, big, "layer, quantizer launch + staged")


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 10000), (2, 4096, 10000), (2, 4096, 9999),
                                   (6, 2048, 10000), (3, 2048, 6144)])
def test_silu_staged(dev, gq, fmt, M, K, N):
    # gate/up pairs: 2N x M x K/256 = 320000 (M = 1: fused from f32, staged from
    # q8_K), 640000 (M = 2: quantizer launch + staged), 960000 (M = 6: the
    # 8-row staged form; 9999 pairs leave a ragged last tile) and 294912 (M = 3,
    # rows of 8 blocks: quantizer launch + staged); the first SUB / 2 outputs
    # equal a small call's (fused or plain) bit for bit
    log("gemv silu staged fmt=%d M=%d" % (fmt, M))
    rng = np.random.default_rng(200 + fmt + M)
    wg = synth.make_weights(rng, fmt, N, K)
    wu = synth.make_weights(rng, fmt, N, K)
    x = to_dev(synth.make_activations(rng, M, K, True))
    y, _ = gq.linear_silu_mul(fmt, to_dev(wg), to_dev(wu), x, N, path=PATH_GEMV)
    n = SUB // 2
    ys, _ = gq.linear_silu_mul(fmt, to_dev(wg[:n]), to_dev(wu[:n]), x, n, path=PATH_GEMV)
    assert np.array_equal(to_host(y)[:, :n].view(np.uint32), to_host(ys).view(np.uint32))
