"""GPU parity for q2_K, q3_K and q5_K (the K-quant rung's other formats).

Every route the library takes for these formats, against the oracle:
  * the device unpacker (gemmq_decode) bit for bit, on random and on extreme
    fields (every scale and min at its limits, d negative, zero, subnormal and
    65504);
  * the GEMV for M = 1..8 over row lengths that select every launch shape
    (P rows a round, two rows a wave, rows split over 2/3/4 waves, two rounds in
    flight), and the bits of a row independent of M;
  * the MFMA GEMM with ragged tiles in M and N, any row subset giving identical
    bits;
  * grouped launches equal to single calls, the whole layer (gemmq_linear_group,
    fused and two-launch) equal to quantize + gemm, and the SiLU-gated pair.
Outputs within 1e-5 * sum_k|w_k * xhat_k| + 1e-6 of the oracle's exact route.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from packer import pack_q2K, pack_q3K, pack_q5K
from quant_packed_weight_amd import synth

pytestmark = pytest.mark.gpu

Q2, Q3, Q5 = 10, 11, 13
FMTS = [Q2, Q3, Q5]


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def _extreme(rng, fmt, n):
    """Blocks whose fields sit at their limits: scales and mins at 0 and at the
    maximum, every quant value, and d/dmin negative, zero, subnormal, 65504."""
    d = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    dmin = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    if n >= 4:
        d[:4] = [-0.5, 0.0, 6e-8, 0.25]
        dmin[:4] = [0.25, -3.0, 6.1e-5, 0.0]
    if fmt == Q2:
        sc, mn = rng.integers(0, 16, (n, 16)), rng.integers(0, 16, (n, 16))
        sc[::3], mn[1::3] = 15, 15
        q = rng.integers(0, 4, (n, 256))
        q[:, ::7] = 3
        return pack_q2K(d, dmin, sc, mn, q)
    if fmt == Q3:
        sc = rng.integers(-32, 32, (n, 16))
        sc[::3] = -32
        sc[1::3] = 31
        q = rng.integers(-4, 4, (n, 256))
        q[:, ::5] = -4
        q[:, 1::5] = 3
        return pack_q3K(d, sc, q)
    sc, mn = rng.integers(0, 64, (n, 8)), rng.integers(0, 64, (n, 8))
    sc[::3], mn[1::3] = 63, 63
    q = rng.integers(0, 32, (n, 256))
    q[:, ::7] = 31
    return pack_q5K(d, dmin, sc, mn, q)


def _case(orc, fmt, M, N, K, seed, extreme=False):
    rng = np.random.default_rng(seed)
    if extreme:
        W = _extreme(rng, fmt, N * (K // 256)).reshape(N, -1)
    else:
        W = synth.make_weights(rng, fmt, N, K)
    x = synth.make_activations(rng, M, K, True)
    if extreme:
        x[:, 0] = np.abs(x).max() * 3  # x = +amax in some blocks, -amax in one
        x[0, 1] = -x[0, 0]
    return W, x, orc.quantize_q8K(x)


def _check(gq, orc, fmt, W, xq, M, N, K, path, where):
    y = to_host(gq.gemm(fmt, to_dev(W), to_dev(xq), M, N, K, path=path))
    yo = orc.gemm_int(fmt, W, xq, M, N, K)
    _, S = orc.gemm_dequant(fmt, W, xq, M, N, K)
    return assert_within(y, yo, S, where)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,extreme", [(1, 256, False), (33, 768, True), (1000, 512, False),
                                         (7, 3072, True), (129, 256, True)])
def test_decode_bit_exact(dev, gq, orc, fmt, N, K, extreme):
    log("decode fmt=%d N=%d K=%d extreme=%d" % (fmt, N, K, extreme))
    W, _, _ = _case(orc, fmt, 1, N, K, seed=N + K + fmt, extreme=extreme)
    got = to_host(gq.decode(fmt, to_dev(W), N, K))
    want = orc.decode(fmt, W, N, K)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# row lengths: 1, 2, 4, 8 blocks (16/8/4/2 rows a round), 3 and 16 (two rows a
# wave), 32 / 48 / 64 (split over 2 / 3 / 4 waves), 80 (two rounds in flight)
GEMV_SHAPES = [(1, 256), (31, 512), (33, 768), (1000, 1024), (64, 2048), (130, 4096),
               (40, 8192), (33, 12288), (9, 16384), (17, 20480)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("N,K", GEMV_SHAPES)
def test_gemv_parity(dev, gq, orc, fmt, M, N, K):
    log("gemv fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    W, _, xq = _case(orc, fmt, M, N, K, seed=100 * M + N + K + fmt)
    _check(gq, orc, fmt, W, xq, M, N, K, gq.PATH_GEMV, "gemv")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [256, 1024, 4096, 12288, 20480])
def test_gemv_rows_independent_of_M(dev, gq, orc, fmt, K):
    log("gemv M-invariance fmt=%d K=%d" % (fmt, K))
    N = 333
    W, _, xq = _case(orc, fmt, 8, N, K, seed=K + fmt)
    Wd = to_dev(W)
    y8 = to_host(gq.gemm(fmt, Wd, to_dev(xq), 8, N, K, path=gq.PATH_GEMV))
    for m in range(8):
        y1 = to_host(gq.gemm(fmt, Wd, to_dev(xq[m:m + 1]), 1, N, K, path=gq.PATH_GEMV))
        assert np.array_equal(y1[0].view(np.uint32), y8[m].view(np.uint32)), m


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(9, 1, 256), (16, 33, 512), (32, 65, 768), (33, 200, 1024),
                                   (128, 64, 512), (129, 127, 256), (300, 130, 1024),
                                   (511, 96, 3072), (1, 70, 512), (40, 70, 8192),
                                   (70, 130, 12544), (600, 1500, 256)])
def test_gemm_parity(dev, gq, orc, fmt, M, N, K):
    log("gemm fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    W, _, xq = _case(orc, fmt, M, N, K, seed=7 * M + 3 * N + K + fmt)
    _check(gq, orc, fmt, W, xq, M, N, K, gq.PATH_GEMM, "gemm")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_rows_independent_of_call(dev, gq, orc, fmt):
    log("gemm row-subset fmt=%d" % fmt)
    M, N, K = 300, 150, 1024
    W, _, xq = _case(orc, fmt, M, N, K, seed=77 + fmt)
    Wd = to_dev(W)
    full = to_host(gq.gemm(fmt, Wd, to_dev(xq), M, N, K, path=gq.PATH_GEMM))
    for a, b in [(0, 9), (37, 87), (128, 300), (299, 300)]:
        part = to_host(gq.gemm(fmt, Wd, to_dev(xq[a:b]), b - a, N, K, path=gq.PATH_GEMM))
        assert np.array_equal(part.view(np.uint32), full[a:b].view(np.uint32)), (a, b)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path,M", [(1, 1), (1, 8), (2, 40)])
def test_extreme_fields(dev, gq, orc, fmt, path, M):
    log("extreme fmt=%d path=%d M=%d" % (fmt, path, M))
    N, K = 70, 1792
    W, _, xq = _case(orc, fmt, M, N, K, seed=5 + fmt, extreme=True)
    _check(gq, orc, fmt, W, xq, M, N, K, path, "extreme")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path,M", [(1, 1), (1, 5), (2, 9), (2, 130)])
def test_group_equals_single_calls(dev, gq, orc, fmt, path, M):
    log("group fmt=%d path=%d M=%d" % (fmt, path, M))
    K = 1024
    Ns = [300, 0, 65, 1000]
    rng = np.random.default_rng(31 * M + fmt + path)
    Ws = [synth.make_weights(rng, fmt, N, K) for N in Ns]
    xq = orc.quantize_q8K(synth.make_activations(rng, M, K, True))
    xqd = to_dev(xq)
    outs = gq.gemm_group(fmt, [to_dev(W) for W in Ws], xqd, M, Ns, K, path=path)
    for W, N, o in zip(Ws, Ns, outs):
        single = to_host(gq.gemm(fmt, to_dev(W), xqd, M, N, K, path=path))
        assert np.array_equal(to_host(o).view(np.uint32), single.view(np.uint32)), N


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,Ns", [(1, 1024, [77, 300]), (4, 4096, [129]), (1, 12288, [70]),
                                    (3, 2048, [40, 9]), (40, 1024, [65])])
def test_linear_equals_quantize_then_gemm(dev, gq, orc, fmt, M, K, Ns):
    # fused at decode shapes (M <= 4, rows of at most 16 blocks), two launches otherwise
    log("linear fmt=%d M=%d K=%d Ns=%s" % (fmt, M, K, Ns))
    rng = np.random.default_rng(1000 * M + K + fmt)
    x = synth.make_activations(rng, M, K, True)
    Ws = [synth.make_weights(rng, fmt, N, K) for N in Ns]
    xd, Wd = to_dev(x), [to_dev(W) for W in Ws]
    outs, xq = gq.linear_group(fmt, Wd, xd, Ns)
    xq_o = orc.quantize_q8K(x)
    assert np.array_equal(to_host(xq).reshape(xq_o.shape), xq_o)
    refs = gq.gemm_group(fmt, Wd, to_dev(xq_o), M, Ns, K)
    for N, o, r in zip(Ns, outs, refs):
        assert np.array_equal(to_host(o).view(np.uint32), to_host(r).view(np.uint32)), N
    yo = orc.gemm_int(fmt, Ws[0], xq_o, M, Ns[0], K)
    _, S = orc.gemm_dequant(fmt, Ws[0], xq_o, M, Ns[0], K)
    assert_within(to_host(outs[0]), yo, S, "linear")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,N", [(1, 2048, 300), (2, 8192, 129), (40, 1024, 200)])
def test_silu_mul(dev, gq, orc, fmt, M, K, N):
    # against the device's own gate/up matmuls: the product of the same G and U
    log("silu fmt=%d M=%d K=%d N=%d" % (fmt, M, K, N))
    rng = np.random.default_rng(7 * M + K + N + fmt)
    x = synth.make_activations(rng, M, K, True)
    Wg, Wu = synth.make_weights(rng, fmt, N, K), synth.make_weights(rng, fmt, N, K)
    wgd, wud = to_dev(Wg), to_dev(Wu)
    y, xq = gq.linear_silu_mul(fmt, wgd, wud, to_dev(x), N)
    G, U = gq.gemm_group(fmt, [wgd, wud], xq, M, [N, N], K)
    G, U = to_host(G).astype(np.float64), to_host(U).astype(np.float64)
    ref = G / (1.0 + np.exp(-np.clip(G, -700, 700))) * U
    y = to_host(y).astype(np.float64)
    bound = 8 * 2.0 ** -24 * np.abs(ref) + np.abs(G * U) * 2.0 ** -126 + 2.0 ** -149
    assert (np.abs(y - ref) <= bound).all()


@pytest.mark.parametrize("fmt", [Q2, Q3, Q5, 12, 14])
@pytest.mark.parametrize("path", [1, 2])
def test_longest_rows(dev, gq, orc, fmt, path):
    # K at the library's limit (2^24, one row of 65536 super-blocks): the GEMV's
    # looping four-wave split and the GEMM's K loop (split in two for q4_K)
    K = 1 << 24
    M, N = (1, 3) if path == 1 else (9, 2)
    log("longest rows fmt=%d path=%d M=%d N=%d K=%d" % (fmt, path, M, N, K))
    rng = np.random.default_rng(fmt + path)
    W = synth.make_weights(rng, fmt, N, K)
    xq = orc.quantize_q8K(synth.make_activations(rng, M, K, True))
    _check(gq, orc, fmt, W, xq, M, N, K, path, "K=2^24")


# 600 rows x 4200 columns: the plane kernel's 128-row grid has 5 x 66 workgroups
# (ragged in both), above 256, so the call runs 128-row tiles; its row subsets
# (1 or 2 row tiles, 66 or 132 workgroups) run the 64-row tiles.  The tile height
# does not enter any output's arithmetic: the bits agree.
@pytest.mark.parametrize("fmt", [Q2, Q3, Q5, 14, 256 + Q3, 256 + 14])
def test_gemm_tile_heights_same_bits(dev, gq, orc, fmt):
    M, N, K = 600, 4200, 512
    base = fmt & 255
    log("gemm tile heights fmt=%d" % fmt)
    W, _, xq = _case(orc, base, M, N, K, seed=91 + fmt)
    Wd = to_dev(W)
    if fmt > 255:
        Wd = gq.repack(base, Wd, N, K)
    full = to_host(gq.gemm(fmt, Wd, to_dev(xq), M, N, K, path=gq.PATH_GEMM))
    for a, b in [(0, 64), (100, 300), (536, 600), (599, 600)]:
        part = to_host(gq.gemm(fmt, Wd, to_dev(xq[a:b]), b - a, N, K, path=gq.PATH_GEMM))
        assert np.array_equal(part.view(np.uint32), full[a:b].view(np.uint32)), (a, b)
    rows = np.array([0, 31, 32, 63, 64, 127, 128, 255, 300, 511, 512, 575, 599])
    yo = orc.gemm_int(base, W, xq, M, N, K, rows)
    _, S = orc.gemm_dequant(base, W, xq, M, N, K, rows)
    assert_within(full[rows], yo, S, "tile heights")


@pytest.mark.parametrize("fmt", [Q2, Q3, Q5, 14])
def test_silu_tile_heights_same_bits(dev, gq, orc, fmt):
    # 2100 gate/up pairs: 66 pair tiles of 64 interleaved columns (the last
    # ragged) over 5 row tiles of 128 for 600 rows; 3-row calls take 64-row tiles
    M, N, K = 600, 2100, 512
    log("silu tile heights fmt=%d" % fmt)
    rng = np.random.default_rng(93 + fmt)
    x = synth.make_activations(rng, M, K, True)
    wg = to_dev(synth.make_weights(rng, fmt, N, K))
    wu = to_dev(synth.make_weights(rng, fmt, N, K))
    y, _ = gq.linear_silu_mul(fmt, wg, wu, to_dev(x), N, path=gq.PATH_GEMM)
    y = to_host(y)
    for a in (0, 130, M - 3):
        ys, _ = gq.linear_silu_mul(fmt, wg, wu, to_dev(x[a:a + 3]), N, path=gq.PATH_GEMM)
        assert np.array_equal(to_host(ys).view(np.uint32), y[a:a + 3].view(np.uint32)), a
