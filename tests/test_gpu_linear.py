"""GPU: the whole linear layer from f32 activations (gemmq_linear_group).

It must give the bits of gemmq_quantize_q8K followed by gemmq_gemm_group, for
the q8_K blocks it writes and for every output, whether it runs as one fused
launch (decode shapes: each workgroup quantizes into its own LDS) or as two.
The q8_K bytes are also checked against the oracle, and one output per case
against the oracle's integer route within 1e-5 * sum_k |w_k * xhat_k| + 1e-6.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from quant_packed_weight_amd import synth

pytestmark = pytest.mark.gpu

Q4, Q6 = 12, 14


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def _acts(rng, M, K, special=False):
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, min(4, K), replace=False)] *= 20
    if special and M * (K // 256) >= 4:
        xb = x.reshape(-1, 256)
        xb[0] = 0  # d = 0: an all-zero block
        xb[1, :254] = ((np.arange(-127, 127) + 0.5) * 2.0 ** -7).astype(np.float32)  # ties
        xb[1, 254] = 127 * 2.0 ** -7
        xb[1, 255] = 0
        xb[2] = np.float32(1e-39) * np.sign(xb[2])  # denormal inputs
        xb[3] = 0
        xb[3, 17] = -3.0  # a single spike
    return x


# (M, K, Ns, path): fused shapes first (GEMV path, rows of at most 16 blocks,
# M <= 4, M K/256 <= 32), then shapes that take two launches (longer rows,
# M > 4, the GEMM path)
CASES = [
    (1, 256, [300, 0, 65], 0),
    (1, 512, [130], 0),
    (1, 1024, [77, 1029], 0),
    (1, 2048, [9], 0),
    (1, 3072, [1000, 1], 0),
    (1, 4096, [1030, 7, 8, 9], 0),
    (1, 8192, [515], 0),
    (1, 12288, [4099], 0),
    (1, 16384, [260], 1),
    (2, 2048, [300], 0),
    (3, 1024, [100, 17], 0),
    (4, 1024, [333], 1),
    (4, 768, [50], 0),
    (2, 4096, [600, 5], 0),
    (4, 2048, [129], 1),
    (1, 4096, [0, 0], 0),       # no matrix: quantizes only
    (1, 12800, [300, 5], 0),    # 50 blocks a row: two launches
    (2, 12288, [40], 0),        # split rows with M = 2: two launches
    (1, 20480, [70], 0),        # 80 blocks a row: two launches
    (2, 8192, [100], 0),        # M K/256 too large to fuse
    (5, 1024, [100, 3], 0),     # M > 4
    (40, 1024, [300, 65], 0),   # GEMM path
    (1, 1024, [200], 2),        # GEMM path forced at M = 1
]


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("M,K,Ns,path", CASES)
def test_linear_equals_quantize_then_gemm(dev, gq, orc, fmt, M, K, Ns, path):
    log("linear fmt=%d M=%d K=%d Ns=%s path=%d" % (fmt, M, K, Ns, path))
    rng = np.random.default_rng(1000 * M + K + 7 * fmt + path + sum(Ns))
    x = _acts(rng, M, K, special=(K == 1024 and M == 1))
    Ws = [synth.make_weights(rng, fmt, N, K) for N in Ns]
    xd = to_dev(x)
    Wd = [to_dev(W) for W in Ws]
    outs, xq = gq.linear_group(fmt, Wd, xd, Ns, path=path)
    xq_ref = gq.quantize_q8K(xd)
    assert np.array_equal(to_host(xq), to_host(xq_ref))
    xq_o = orc.quantize_q8K(x)
    assert np.array_equal(to_host(xq).reshape(xq_o.shape), xq_o)
    refs = gq.gemm_group(fmt, Wd, xq_ref, M, Ns, K, path=path)
    for N, o, r in zip(Ns, outs, refs):
        assert np.array_equal(to_host(o).view(np.uint32), to_host(r).view(np.uint32)), N
    g = max(range(len(Ns)), key=lambda i: Ns[i])
    if Ns[g] > 0:
        yo = orc.gemm_int(fmt, Ws[g], xq_o, M, Ns[g], K)
        _, S = orc.gemm_dequant(fmt, Ws[g], xq_o, M, Ns[g], K)
        assert_within(to_host(outs[g]), yo, S, "linear")


def test_linear_repeated_calls_reuse_buffers(dev, gq):
    # the same output and q8_K buffers across calls of different shapes: every
    # call overwrites them fully (no stale LDS or global state between launches)
    import torch

    rng = np.random.default_rng(5)
    K = 4096
    W = to_dev(synth.make_weights(rng, Q4, 1000, K))
    xq = torch.zeros((4, (K // 256) * 292), dtype=torch.uint8, device="cuda:0")
    out = torch.full((4, 1000), float("nan"), dtype=torch.float32, device="cuda:0")
    for M in (1, 4, 2, 1):
        x = to_dev(_acts(rng, M, K))
        o, q = gq.linear_group(Q4, [W], x, [1000], xq=xq[:M], outs=[out[:M]])
        ref = gq.gemm(Q4, W, gq.quantize_q8K(x), M, 1000, K)
        assert np.array_equal(to_host(o[0]).view(np.uint32), to_host(ref).view(np.uint32)), M
        assert np.array_equal(to_host(q), to_host(gq.quantize_q8K(x))), M
