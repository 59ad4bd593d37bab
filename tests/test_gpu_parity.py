"""GPU parity: the HIP path against the CPU oracle, element by element.

Bit-exact: q8_K bytes and decoded weights.  Tolerance: |y - y_oracle| <=
1e-5 * sum_k |w_k * xhat_k| + 1e-6 per output (the pages' 1e-5 scaled relative
bound for reordered f32 sums; molayo article, status row "src/ -- C++ engine").
Bit identity inside a path: GEMV rows do not depend on M, GEMM rows do not
depend on which other rows are in the call (the pages' tiled equals single-row
rule, same row of the article).
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev, to_host
from packer import pack_q4K, pack_q6K
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


def _acts(rng, M, K, kind="normal"):
    x = rng.standard_normal((M, K)).astype(np.float32)
    if kind == "outliers" and K >= 4:
        x[:, rng.choice(K, 4, replace=False)] *= 20
    return x


# ------------------------------------------------------------------ q8_K
@pytest.mark.parametrize("M,K", [(1, 256), (3, 768), (8, 4096), (37, 1024), (512, 2048),
                                 (2, 12288)])
def test_quantize_bit_exact(dev, gq, orc, M, K):
    log("quantize M=%d K=%d" % (M, K))
    rng = np.random.default_rng(M * 7 + K)
    x = _acts(rng, M, K, "outliers")
    # special blocks: all zero, exact ties, tiny values, a single spike
    nb = K // 256
    if M * nb >= 4:
        xb = x.reshape(-1, 256)
        xb[0] = 0
        # d = 2^-7 exactly, so x/d hits every k + 1/2 tie exactly
        xb[1, :254] = ((np.arange(-127, 127) + 0.5) * 2.0 ** -7).astype(np.float32)
        xb[1, 254] = 127 * 2.0 ** -7
        xb[1, 255] = 0
        xb[2] = np.float32(1e-39) * np.sign(xb[2])
        xb[3] = 0
        xb[3, 17] = -3.0
    got = to_host(gq.quantize_q8K(to_dev(x)))
    want = orc.quantize_q8K(x)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ decode
def _adversarial_q4K(rng, n):
    d = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    dmin = (np.abs(rng.standard_normal(n)) * 2e-3).astype(np.float16)
    sc = rng.integers(0, 64, (n, 8))
    mn = rng.integers(0, 64, (n, 8))
    q = rng.integers(0, 16, (n, 256))
    d[0::7] = np.float16(6e-8)     # f16 subnormal
    dmin[1::7] = np.float16(3e-6)  # f16 subnormal
    d[2::7] = 0
    d[3::7] = -d[3::7]             # negative scales
    dmin[4::7] = -np.float16(0.5)
    sc[5::7] = 63
    mn[5::7] = 63
    q[5::7] = 15
    d[6::7] = np.float16(65504.0)
    return pack_q4K(d, dmin, sc, mn, q)


def _adversarial_q6K(rng, n):
    d = (np.abs(rng.standard_normal(n)) * 1e-3).astype(np.float16)
    sc = rng.integers(-128, 128, (n, 16))
    q = rng.integers(0, 64, (n, 256))
    d[0::5] = np.float16(6e-8)
    d[1::5] = 0
    d[2::5] = -d[2::5]
    sc[3::5] = -128
    q[3::5] = 0  # (0 - 32) * -128 = 4096, the largest magnitude
    sc[4::5] = 127
    q[4::5] = 63
    return pack_q6K(d, sc, q)


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("N,K", [(1, 256), (33, 768), (1000, 512), (7, 3072)])
def test_decode_bit_exact(dev, gq, orc, fmt, N, K):
    log("decode fmt=%d N=%d K=%d" % (fmt, N, K))
    rng = np.random.default_rng(N + K + fmt)
    nb = K // 256
    if N * nb >= 10:
        raw = (_adversarial_q4K if fmt == Q4 else _adversarial_q6K)(rng, N * nb).reshape(N, -1)
    else:
        raw = synth.make_weights(rng, fmt, N, K)
    got = to_host(gq.decode(fmt, to_dev(raw), N, K))
    want = orc.decode(fmt, raw, N, K)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------------ matmul
def _case(orc, fmt, M, N, K, seed, adversarial=False):
    rng = np.random.default_rng(seed)
    nb = K // 256
    if adversarial:
        W = (_adversarial_q4K if fmt == Q4 else _adversarial_q6K)(rng, N * nb).reshape(N, -1)
    else:
        W = synth.make_weights(rng, fmt, N, K)
    x = _acts(rng, M, K, "outliers")
    if adversarial:
        x[:, 0] = np.abs(x).max() * 3  # x = +amax in some blocks
        x[0, 1] = -x[0, 0]            # and -amax
    xq = orc.quantize_q8K(x)
    return W, x, xq


def _run(gq, fmt, W, xq, M, N, K, path):
    return to_host(gq.gemm(fmt, to_dev(W), to_dev(xq), M, N, K, path=path))


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", [(1, 256), (31, 512), (33, 768), (1000, 1024), (64, 3072),
                                 (40, 8192), (33, 12288), (17, 20480)])
def test_gemv_parity(dev, gq, orc, fmt, M, N, K):
    log("gemv fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    W, _, xq = _case(orc, fmt, M, N, K, seed=100 * M + N + K + fmt)
    y = _run(gq, fmt, W, xq, M, N, K, gq.PATH_GEMV)
    yo = orc.gemm_int(fmt, W, xq, M, N, K)
    _, S = orc.gemm_dequant(fmt, W, xq, M, N, K)
    assert_within(y, yo, S, "gemv")


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("K", [256, 1024, 3072, 4096, 12288, 20480])
def test_gemv_rows_independent_of_M(dev, gq, orc, fmt, K):
    log("gemv M-invariance fmt=%d K=%d" % (fmt, K))
    N = 333
    W, _, xq = _case(orc, fmt, 8, N, K, seed=K + fmt)
    Wd = to_dev(W)
    y8 = to_host(gq.gemm(fmt, Wd, to_dev(xq), 8, N, K, path=gq.PATH_GEMV))
    for m in range(8):
        y1 = to_host(gq.gemm(fmt, Wd, to_dev(xq[m:m + 1]), 1, N, K, path=gq.PATH_GEMV))
        assert np.array_equal(y1[0].view(np.uint32), y8[m].view(np.uint32)), m
    for M in (3, 5):
        yM = to_host(gq.gemm(fmt, Wd, to_dev(xq[:M]), M, N, K, path=gq.PATH_GEMV))
        assert np.array_equal(yM.view(np.uint32), y8[:M].view(np.uint32))


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("M,N,K", [(9, 1, 256), (16, 33, 512), (31, 64, 256), (32, 65, 768),
                                   (33, 200, 1024), (128, 64, 512), (129, 127, 256),
                                   (300, 130, 1024), (511, 96, 3072), (1, 70, 512), (8, 64, 256),
                                   (40, 70, 8192), (70, 130, 12544), (600, 4500, 256)])
def test_gemm_parity(dev, gq, orc, fmt, M, N, K):
    log("gemm fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    W, _, xq = _case(orc, fmt, M, N, K, seed=7 * M + 3 * N + K + fmt)
    y = _run(gq, fmt, W, xq, M, N, K, gq.PATH_GEMM)
    yo = orc.gemm_int(fmt, W, xq, M, N, K)
    _, S = orc.gemm_dequant(fmt, W, xq, M, N, K)
    assert_within(y, yo, S, "gemm")


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("K", [1024, 8192])
def test_gemm_rows_independent_of_call(dev, gq, orc, fmt, K):
    log("gemm row-subset fmt=%d K=%d" % (fmt, K))
    M, N = 300, 150
    W, _, xq = _case(orc, fmt, M, N, K, seed=77 + fmt)
    Wd = to_dev(W)
    full = to_host(gq.gemm(fmt, Wd, to_dev(xq), M, N, K, path=gq.PATH_GEMM))
    for a, b in [(0, 9), (37, 87), (128, 300), (299, 300), (5, 6)]:
        part = to_host(gq.gemm(fmt, Wd, to_dev(xq[a:b]), b - a, N, K, path=gq.PATH_GEMM))
        assert np.array_equal(part.view(np.uint32), full[a:b].view(np.uint32)), (a, b)


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("path", [1, 2])
def test_adversarial_blocks(dev, gq, orc, fmt, path):
    log("adversarial fmt=%d path=%d" % (fmt, path))
    M = 8 if path == 1 else 40
    N, K = 70, 1792
    W, _, xq = _case(orc, fmt, M, N, K, seed=5 + fmt, adversarial=True)
    y = _run(gq, fmt, W, xq, M, N, K, path)
    yo = orc.gemm_int(fmt, W, xq, M, N, K)
    _, S = orc.gemm_dequant(fmt, W, xq, M, N, K)
    assert_within(y, yo, S, "adversarial")


def _expected_path(gq, fmt, M, cols, K):
    # GEMV up to M = 8 (q4_K: up to 2); the small-M MFMA kernels for q4_K at
    # 3 <= M <= 64 with one 16-row tile, or with t tiles while cols * t <= 20480,
    # and for q6_K at 9 <= M <= 16, or at 3 <= M <= 8 from 16384 columns unless
    # the GEMV holds the activation in LDS (M <= 4, M K/256 <= 32); q4_K at
    # M = 3, 4 also stays on the GEMV where it stages the activation (rows of
    # <= 16 blocks, M K/256 <= 64, cols x M x K/256 >= 2^18); plain q6_K at
    # 5 <= M <= 8 on rows of more than 8 blocks also from cols x K/256 = 2^16,
    # and at M = 3, 4 on rows of more than 64 blocks from 2^18; the GEMM otherwise
    t = (M + 15) // 16
    nb = K // 256
    if fmt == Q4 and M <= 4 and nb <= 16 and M * nb <= 64 and cols * M * nb >= 1 << 18:
        return gq.PATH_GEMV  # the GEMV holds the activation in LDS
    if fmt == Q4 and 3 <= M <= 64 and (t == 1 or cols * t <= 20480):
        return gq.PATH_SKINNY
    staged = M <= 4 and M * (K // 256) <= 32
    if fmt == Q6 and 3 <= M <= 16 and (M > 8 or (cols >= 16384 and not staged)):
        return gq.PATH_SKINNY
    if fmt == Q6 and 5 <= M <= 8 and nb > 8 and cols * nb >= 1 << 16:
        return gq.PATH_SKINNY
    if fmt == Q6 and 3 <= M <= 4 and nb > 64 and cols * nb >= 1 << 18:
        return gq.PATH_SKINNY
    return gq.PATH_GEMV if M <= 8 else gq.PATH_GEMM


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("N", [96, 7000, 16383, 16384])
def test_auto_dispatch_and_linear(dev, gq, orc, fmt, N):
    # the automatic path takes the expected kernel family (the same bits as that
    # path forced); N = 7000 crosses the q4_K column bound between t = 2 and
    # t = 3, N = 16384 the q6_K one at M = 5..8 (M = 3, 4 stay on the GEMV)
    log("dispatch fmt=%d N=%d" % (fmt, N))
    K = 512 if N < 1000 else 256
    for M in (1, 2, 3, 4, 5, 6, 8, 9, 16, 17, 32, 33, 48, 49, 64, 65):
        W, x, xq = _case(orc, fmt, M, N, K, seed=M + fmt)
        auto = to_host(gq.gemm(fmt, to_dev(W), to_dev(xq), M, N, K))
        path = _expected_path(gq, fmt, M, N, K)
        forced = _run(gq, fmt, W, xq, M, N, K, path)
        assert np.array_equal(auto.view(np.uint32), forced.view(np.uint32)), M
        lin = to_host(gq.linear(fmt, to_dev(W), to_dev(x), N))
        assert np.array_equal(lin.view(np.uint32), auto.view(np.uint32)), M


@pytest.mark.parametrize("M,K,N", [(5, 4096, 4096), (8, 4096, 4095), (6, 2304, 7282),
                                   (8, 2304, 7281), (8, 2048, 8192), (3, 4096, 8192),
                                   (8, 12288, 1366), (3, 16640, 4034), (4, 16640, 4032),
                                   (4, 16384, 8192)])
def test_auto_dispatch_q6K_long_rows(dev, gq, orc, M, K, N):
    # plain q6_K at M = 5..8 on rows of more than 8 blocks takes the small-M
    # kernel from output columns x K/256 = 2^16, at M = 3, 4 on rows of more
    # than 64 blocks from 2^18 (each pair of cases straddles a bound); rows of
    # 8 blocks, and of 64 at M = 3, 4, keep the GEMV.  The automatic path
    # equals the expected path forced, and sampled outputs the oracle.
    log("dispatch q6_K long rows M=%d K=%d N=%d" % (M, K, N))
    W, x, xq = _case(orc, Q6, M, N, K, seed=M + K + N)
    auto = to_host(gq.gemm(Q6, to_dev(W), to_dev(xq), M, N, K))
    path = _expected_path(gq, Q6, M, N, K)
    nb = K // 256
    want = (5 <= M <= 8 and nb > 8 and N * nb >= 1 << 16) or (
        3 <= M <= 4 and nb > 64 and N * nb >= 1 << 18)
    assert (path == gq.PATH_SKINNY) == want
    forced = _run(gq, Q6, W, xq, M, N, K, path)
    assert np.array_equal(auto.view(np.uint32), forced.view(np.uint32))
    cols = np.array([0, N // 3, N // 2, N - 1])
    Ws = np.ascontiguousarray(W[cols])
    yo = orc.gemm_int(Q6, Ws, xq, M, len(cols), K)
    _, S = orc.gemm_dequant(Q6, Ws, xq, M, len(cols), K)
    assert_within(auto[:, cols], yo, S, "q6_K long rows, automatic path")


@pytest.mark.parametrize("M,K,N", [(3, 4096, 30000), (4, 4096, 30000), (4, 2048, 8192),
                                   (3, 4096, 300), (3, 12288, 30000), (8, 4096, 30000)])
def test_auto_dispatch_q4K_large_launches(dev, gq, orc, M, K, N):
    # q4_K at M = 3, 4 stays on the GEMV where it holds the activation in LDS
    # (large launches of rows of <= 16 blocks); small launches, long rows and
    # M > 4 keep the small-M kernel.  The automatic path, the one-call layer and
    # that path forced give the same bits; sampled outputs match the oracle.
    log("dispatch q4_K large M=%d K=%d N=%d" % (M, K, N))
    W, x, xq = _case(orc, Q4, M, N, K, seed=M + K + N)
    Wd, xqd = to_dev(W), to_dev(xq)
    auto = to_host(gq.gemm(Q4, Wd, xqd, M, N, K))
    path = _expected_path(gq, Q4, M, N, K)
    forced = _run(gq, Q4, W, xq, M, N, K, path)
    assert np.array_equal(auto.view(np.uint32), forced.view(np.uint32))
    lin = to_host(gq.linear(Q4, Wd, to_dev(x), N))
    assert np.array_equal(lin.view(np.uint32), auto.view(np.uint32))
    cols = np.array([0, 1, N // 3, N // 2, N - 2, N - 1])
    Ws = np.ascontiguousarray(W[cols])
    yo = orc.gemm_int(Q4, Ws, xq, M, len(cols), K)
    _, S = orc.gemm_dequant(Q4, Ws, xq, M, len(cols), K)
    assert_within(auto[:, cols], yo, S, "q4_K large dispatch")


@pytest.mark.parametrize("N", [16383, 16384])
def test_auto_dispatch_q6K_repacked(dev, gq, orc, N):
    # the repacked q6_K layout follows the q6_K choice (the small-M kernel at
    # M = 9..16 and at 5..8 from 16384 columns, the GEMV below, the GEMM beyond)
    # with the original layout's bits
    import torch

    K = 512
    for M in (2, 4, 5, 8, 16, 17):
        log("dispatch q6_K_R N=%d M=%d" % (N, M))
        W, x, xq = _case(orc, Q6, M, N, K, seed=100 + M)
        Wd, xqd = to_dev(W), to_dev(xq)
        Wr = gq.repack(Q6, Wd, N, K)
        auto = to_host(gq.gemm(gq.FMT_Q6K_R, Wr, xqd, M, N, K))
        path = _expected_path(gq, Q6, M, N, K)
        forced = to_host(gq.gemm(gq.FMT_Q6K_R, Wr, xqd, M, N, K, path=path))
        plain = to_host(gq.gemm(Q6, Wd, xqd, M, N, K, path=path))
        assert np.array_equal(auto.view(np.uint32), forced.view(np.uint32)), M
        assert np.array_equal(auto.view(np.uint32), plain.view(np.uint32)), M
        torch.cuda.synchronize()


def test_empty_calls_touch_nothing(dev, gq):
    import torch

    y = torch.full((4, 4), 7.0, device="cuda:0")
    w = torch.zeros(4 * 144, dtype=torch.uint8, device="cuda:0")
    xq = torch.zeros(4 * 292, dtype=torch.uint8, device="cuda:0")
    assert gq.gemm_ptr(Q4, w.data_ptr(), xq.data_ptr(), y.data_ptr(), 0, 4, 256) == 0
    assert gq.gemm_ptr(Q4, w.data_ptr(), xq.data_ptr(), y.data_ptr(), 4, 0, 256) == 0
    for path in (gq.PATH_GEMV, gq.PATH_SKINNY, gq.PATH_GEMM):
        assert gq.gemm_ptr(Q4, w.data_ptr(), xq.data_ptr(), y.data_ptr(), 0, 4, 256, path) == 0
        assert gq.gemm_ptr(Q4, w.data_ptr(), xq.data_ptr(), y.data_ptr(), 4, 0, 256, path) == 0
    assert gq.quantize_q8K_ptr(y.data_ptr(), xq.data_ptr(), 0, 256) == 0
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    assert bool((xq == 0).all())


def test_quantize_near_ties(dev, gq, orc):
    # values whose x/d lies a little above, below or exactly on k + 1/2, with
    # scales that are not powers of two: the quantizer's rounding must agree
    # with the correctly rounded division everywhere, on both sides of a tie
    log("quantize near ties")
    rng = np.random.default_rng(77)
    M, K = 6, 2048
    x = np.empty((M, K), dtype=np.float32)
    xb = x.reshape(-1, 256)
    deltas = np.array([0, 2.0 ** -9, -2.0 ** -9, 2.0 ** -11, -2.0 ** -11, 2.0 ** -12,
                       -2.0 ** -12, 2.0 ** -13, -2.0 ** -13, 2.0 ** -16, -2.0 ** -16,
                       2.0 ** -20, -2.0 ** -20, 1e-7, -1e-7])
    for i in range(xb.shape[0]):
        amax = np.float32(rng.uniform(0.01, 50.0) if i % 5 else 3e-37)  # one tiny scale in 5
        d = np.float32(amax / np.float32(127))
        k = rng.integers(-127, 127, size=255)
        dl = deltas[rng.integers(0, len(deltas), size=255)]
        vals = ((k + 0.5 + dl) * np.float64(d)).astype(np.float32)
        vals = np.clip(vals, -amax, amax)
        xb[i, :255] = vals
        xb[i, 255] = amax if i % 2 else -amax
    got = to_host(gq.quantize_q8K(to_dev(x)))
    want = orc.quantize_q8K(x)
    assert np.array_equal(got.reshape(want.shape), want)


@pytest.mark.parametrize("fmt", [Q4, Q6])
@pytest.mark.parametrize("path,M", [(1, 1), (1, 5), (2, 9), (2, 130)])
def test_group_equals_single_calls(dev, gq, orc, fmt, path, M):
    # one launch over several matrices sharing the activations gives each matrix
    # the bits of its own call; an empty entry is skipped
    log("group fmt=%d path=%d M=%d" % (fmt, path, M))
    K = 1024
    Ns = [300, 0, 65, 1000]
    rng = np.random.default_rng(31 * M + fmt + path)
    Ws = [synth.make_weights(rng, fmt, N, K) for N in Ns]
    xq = orc.quantize_q8K(_acts(rng, M, K, "outliers"))
    xqd = to_dev(xq)
    outs = gq.gemm_group(fmt, [to_dev(W) for W in Ws], xqd, M, Ns, K, path=path)
    for W, N, o in zip(Ws, Ns, outs):
        single = to_host(gq.gemm(fmt, to_dev(W), xqd, M, N, K, path=path))
        assert np.array_equal(to_host(o).view(np.uint32), single.view(np.uint32)), N
    yo = orc.gemm_int(fmt, Ws[2], xq, M, Ns[2], K)
    _, S = orc.gemm_dequant(fmt, Ws[2], xq, M, Ns[2], K)
    assert_within(to_host(outs[2]), yo, S, "group")
