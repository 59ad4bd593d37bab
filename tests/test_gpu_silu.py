"""GPU: the gated up-projection silu(Wg x) * (Wu x) in one call
(gemmq_linear_silu_mul), on every route: the fused quantize + GEMV launch, the
plain GEMV (long rows, M up to 8), the small-M MFMA kernel (q4_K, M 4..32),
the MFMA GEMM with and without the split K loop, ragged tiles, and N = 0.

Three checks per case:
  * the q8_K bytes equal the oracle's quantizer, bit for bit;
  * against the oracle, y_o = silu(g_o) u_o in float64 from the oracle's exact
    integer route: with the matmul bound d = 1e-5 S + 1e-6 on g and u and
    |silu'| < 1.1,  |y - y_o| <= 1.1 dg (|u_o| + du) + |silu(g_o)| du + 8 ulp;
  * against the device's own matmuls on the same q8_K input (gemmq_gemm_group
    on the gate and the up matrix): y equals silu(G) U for those G, U to within
    the f32 roundings of the product (8 ulp), which a swapped or misaligned
    gate/up pair, or a different G or U, would miss by far.
Both bounds add the f32 range limits: for g < -88.72, exp(-g) overflows and
the f32 form gives +-0 where |silu(g) u| < |g u| / FLT_MAX < |g u| 2^-126 (the
q6_K gates reach -100 here), and a result below 2^-126 is rounded to 2^-149.
"""
import numpy as np
import pytest

from gpu_util import device, log, to_dev, to_host
from quant_packed_weight_amd import synth

pytestmark = pytest.mark.gpu

Q4, Q6 = 12, 14
ULP8 = 8 * 2.0 ** -24  # eight f32 roundings, relative


def _range(g, u):
    """What the f32 range costs: exp(-g) overflowing, and subnormal results."""
    return np.abs(g * u) * 2.0 ** -126 + 2.0 ** -149


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def _silu64(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-np.clip(g, -700, 700)))


# (M, K, N, path, x scale): fused shapes (M <= 4, rows of at most 16 blocks,
# M K/256 <= 32), then plain GEMV shapes, then the GEMM path
CASES = [
    (1, 256, 300, 0, 1.0),
    (1, 1024, 77, 0, 4.0),       # four rows a wave
    (1, 2048, 1029, 0, 1.0),     # two rows a wave, ragged tail
    (1, 4096, 1030, 0, 8.0),     # two rows side by side; saturated gates
    (2, 2048, 300, 0, 1.0),
    (3, 768, 50, 0, 2.0),
    (4, 1024, 333, 0, 1.0),
    (1, 4096, 0, 0, 1.0),        # no output: quantizes only
    (1, 8192, 515, 0, 1.0),      # split rows (two waves a row)
    (1, 12288, 4099, 0, 1.0),    # three waves a row (the down projection's row length)
    (1, 20480, 70, 0, 1.0),      # two rounds in flight, four waves a row
    (5, 1024, 100, 0, 1.0),      # M > 4: two launches
    (8, 4096, 257, 1, 1.0),      # GEMV forced at its largest M
    (2, 8192, 129, 1, 1.0),
    (9, 1024, 65, 0, 1.0),       # automatic path: q4_K small-M MFMA kernel, q6_K GEMM
    (30, 2048, 40, 0, 1.0),      # q4_K: small-M MFMA kernel, two row tiles a wave
    (8, 4096, 257, 0, 1.0),      # q4_K: small-M MFMA kernel (eight waves a row)
    (16, 12288, 70, 0, 2.0),     # q4_K: small-M MFMA kernel, two super-blocks a wave
    (5, 256, 1, 0, 1.0),         # q4_K: small-M MFMA kernel, one output column
    (40, 1024, 300, 0, 2.0),     # q4_K: small-M MFMA kernel, three row tiles; q6_K: GEMM
    (64, 2048, 77, 0, 1.0),      # q4_K: small-M MFMA kernel, four row tiles
    (20, 1024, 11000, 0, 1.0),   # q4_K: 2 x 11000 columns in two row tiles -> GEMM
    (6, 1024, 8200, 0, 1.0),     # q6_K: 2 x 8200 columns at M = 6 -> GEMM
    (40, 1024, 300, 2, 2.0),     # GEMM forced: ragged last tile
    (70, 1024, 300, 0, 1.0),     # GEMM: ragged last tile
    (130, 4096, 200, 0, 1.0),    # several row tiles of M
    (70, 8192, 129, 0, 1.0),     # split K loop
    (17, 256, 1, 0, 1.0),        # one output column
    (1, 1024, 200, 2, 1.0),      # GEMM forced at M = 1
    (40, 1024, 0, 0, 1.0),
]


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("M,K,N,path,scale", CASES)
def test_silu_mul(dev, gq, orc, fmt, M, K, N, path, scale):
    log("silu_mul fmt=%d M=%d K=%d N=%d path=%d" % (fmt, M, K, N, path))
    rng = np.random.default_rng(31 * M + K + 5 * fmt + N + path)
    x = synth.make_activations(rng, M, K, True) * np.float32(scale)
    Wg = synth.make_weights(rng, fmt, N, K)
    Wu = synth.make_weights(rng, fmt, N, K)
    xd, wgd, wud = to_dev(x), to_dev(Wg), to_dev(Wu)
    y, xq = gq.linear_silu_mul(fmt, wgd, wud, xd, N, path=path)
    xq_o = orc.quantize_q8K(x)
    assert np.array_equal(to_host(xq).reshape(xq_o.shape), xq_o)
    if N == 0:
        return
    y = to_host(y).astype(np.float64)
    assert np.all(np.isfinite(y))

    # against the device's own matmuls on the same q8_K input
    G, U = gq.gemm_group(fmt, [wgd, wud], xq, M, [N, N], K, path=path)
    G, U = to_host(G).astype(np.float64), to_host(U).astype(np.float64)
    yd = _silu64(G) * U
    err = np.abs(y - yd)
    bound = ULP8 * np.abs(yd) + _range(G, U)
    assert (err <= bound).all(), ("device", np.argmax(err / bound), float((err / bound).max()))

    # against the oracle
    go = orc.gemm_int(fmt, Wg, xq_o, M, N, K)
    uo = orc.gemm_int(fmt, Wu, xq_o, M, N, K)
    _, Sg = orc.gemm_dequant(fmt, Wg, xq_o, M, N, K)
    _, Su = orc.gemm_dequant(fmt, Wu, xq_o, M, N, K)
    yo = orc.silu_mul(go, uo)
    dg, du = 1e-5 * Sg + 1e-6, 1e-5 * Su + 1e-6
    bound = (1.1 * dg * (np.abs(uo) + du) + np.abs(_silu64(go)) * du + ULP8 * np.abs(yo)
             + _range(np.abs(go) + dg, np.abs(uo) + du))
    err = np.abs(y - yo)
    i = np.unravel_index(np.argmax(err / bound), err.shape)
    log("  max|g| %.3g  worst err/bound %.3g" % (np.abs(go).max(), (err / bound)[i]))
    assert (err <= bound).all(), ("oracle", i, y[i], yo[i], go[i], uo[i])


def test_silu_mul_reuses_buffers(dev, gq):
    # one output and q8_K buffer across calls of different M and routes: every
    # call overwrites them fully
    import torch

    rng = np.random.default_rng(8)
    K, N = 4096, 700
    wg = to_dev(synth.make_weights(rng, Q4, N, K))
    wu = to_dev(synth.make_weights(rng, Q4, N, K))
    xq = torch.zeros((64, (K // 256) * 292), dtype=torch.uint8, device="cuda:0")
    out = torch.full((64, N), float("nan"), dtype=torch.float32, device="cuda:0")
    for M in (1, 4, 64, 2, 1):
        x = to_dev(synth.make_activations(rng, M, K, True))
        y, q = gq.linear_silu_mul(Q4, wg, wu, x, N, xq=xq[:M], out=out[:M])
        y2, _ = gq.linear_silu_mul(Q4, wg, wu, x, N)
        assert np.array_equal(to_host(y).view(np.uint32), to_host(y2).view(np.uint32)), M
        assert np.array_equal(to_host(q), to_host(gq.quantize_q8K(x))), M
