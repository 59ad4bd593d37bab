"""GPU parity in the exact-integer regime: every path must equal the oracle bit
for bit.

With power-of-two weight scales (d, dmin) and power-of-two activation scales
d_x, every term d*sc*q*d_x*q_x and dmin*m*d_x*q_x is an integer multiple of
G = 2^-19 (d, dmin >= 2^-11, d_x >= 2^-8).  When the sum of the terms' magnitudes
stays below 2^23 * G, every partial sum any kernel can form -- in any order, in
int32 or in f32, per sub-block, per super-block or across them, before or after
the d_x factor -- is an exact f32 value, so the f32 result is exact whatever the
summation order and must equal the oracle's exact value (rounded to f32, which
changes nothing).  This reaches each kernel's own unpack (scale/min extraction,
plane folding, repacked loads, the q6_K and q3_K offsets folded through the
group sums) with no tolerance at all: a wrong bit anywhere shows.

The activations are handed over as q8_K blocks built here (any valid blocks
are accepted: |q| <= 127, sums equal to the sums of q); the one-call layer is
fed f32 values the quantizer reproduces exactly (one +-127 per block fixes
d_x = amax/127 to the intended power of two).
"""
import numpy as np
import pytest

from gpu_util import device, log, to_dev, to_host
from packer import pack_q2K, pack_q3K, pack_q4K, pack_q5K, pack_q6K

pytestmark = pytest.mark.gpu

Q2, Q3, Q4, Q5, Q6 = 10, 11, 12, 13, 14
R = 256  # repacked layout: type id + 256
ALL = [Q2, Q3, Q4, Q5, Q6, R + Q3, R + Q6]
PATH_AUTO, PATH_GEMV, PATH_GEMM, PATH_SKINNY = 0, 1, 2, 3
G = 2.0 ** -19          # granularity of every term
LIMIT = 2.0 ** 23 * G   # bound on the sum of the terms' magnitudes


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.fixture(scope="module")
def gq():
    import quant_packed_weight_amd

    return quant_packed_weight_amd


def exact_weights(rng, fmt, N, K, quiet=None):
    """Packed weights with power-of-two d/dmin and full-range fields; returns
    (raw [N, row bytes], mag [N, K]) where mag bounds, per weight, every integer
    product a kernel forms from it (times its power-of-two scale).  `quiet`:
    positions within each block (one per block) whose quant makes sc*q zero in
    every row (q = 0; q6_K: q = 32)."""
    base = fmt & 255
    n = N * (K // 256)

    def hush(q, zero):
        if quiet is not None:
            q.reshape(N, K // 256, 256)[:, np.arange(K // 256), quiet] = zero
        return q

    d = 2.0 ** -rng.integers(10, 12, n)
    dmin = 2.0 ** -rng.integers(10, 12, n)
    if base in (Q4, Q5):
        sc, mn = rng.integers(0, 64, (n, 8)), rng.integers(0, 64, (n, 8))
        q = hush(rng.integers(0, 16 if base == Q4 else 32, (n, 256)), 0)
        raw = (pack_q4K if base == Q4 else pack_q5K)(d, dmin, sc, mn, q)
        mag = d[:, None] * np.repeat(sc, 32, 1) * q + dmin[:, None] * np.repeat(mn, 32, 1)
    elif base == Q2:
        sc, mn = rng.integers(0, 16, (n, 16)), rng.integers(0, 16, (n, 16))
        q = hush(rng.integers(0, 4, (n, 256)), 0)
        raw = pack_q2K(d, dmin, sc, mn, q)
        mag = d[:, None] * np.repeat(sc, 16, 1) * q + dmin[:, None] * np.repeat(mn, 16, 1)
    elif base == Q3:
        sc, q = rng.integers(-32, 32, (n, 16)), hush(rng.integers(-4, 4, (n, 256)), 0)
        raw = pack_q3K(d, sc, q)
        # the -4 of a clear mask bit is folded in int32 (exact), so the f32
        # terms are subset sums of the weights' own products
        mag = d[:, None] * np.abs(np.repeat(sc, 16, 1) * q)
    else:
        sc, q = rng.integers(-128, 128, (n, 16)), hush(rng.integers(0, 64, (n, 256)), 32)
        raw = pack_q6K(d, sc, q)
        # the -32 offset is folded in int32 (exact), as for q3_K
        mag = d[:, None] * np.abs(np.repeat(sc, 16, 1) * (q - 32))
    return raw.reshape(N, -1), mag.reshape(N, K)


def exact_acts(rng, M, K, mag, spike=None):
    """q8_K fields (dx [M, nb], qx [M, K] int) whose every output stays within
    LIMIT for the weight magnitudes `mag`; spike: per block, the position (as
    given to exact_weights' `quiet`) that holds a +-127 in every row."""
    nb = K // 256
    dx = 2.0 ** -rng.integers(7, 9, (M, nb))
    u = rng.random((M, K))
    qx = np.where(u < 0.5, 0, rng.integers(1, 8, (M, K)))
    qx = np.where(u > 0.97, rng.integers(8, 127, (M, K)), qx)
    qx = qx * rng.choice([-1, 1], (M, K))
    spikes = None
    if spike is not None:
        spikes = np.repeat((np.asarray(spike) + 256 * np.arange(nb))[None, :], M, 0)
        np.put_along_axis(qx, spikes, rng.choice([-127, 127], (M, nb)), axis=1)
    dxk = np.repeat(dx, 256, 1)
    for m in range(M):
        while True:
            B = (mag * (dxk[m] * np.abs(qx[m]))[None, :]).sum(1).max()
            if B <= LIMIT:
                break
            nz = np.flatnonzero(qx[m])
            if spike is not None:
                nz = np.setdiff1d(nz, spikes[m])
            assert nz.size, "the spikes alone pass the bound; use a shorter K"
            qx[m, rng.choice(nz, (nz.size + 1) // 2, replace=False)] = 0
    return dx, qx


def q8K_bytes(dx, qx):
    M, K = qx.shape
    nb = K // 256
    out = np.zeros((M, nb, 292), np.uint8)
    q = qx.reshape(M, nb, 256)
    out[:, :, 0:4] = dx.astype(np.float32).reshape(M, nb, 1).view(np.uint8)
    out[:, :, 4:260] = q.astype(np.int8).view(np.uint8)
    s = q.reshape(M, nb, 16, 16).sum(3).astype(np.int16)
    out[:, :, 260:292] = s.view(np.uint8).reshape(M, nb, 32)
    return out.reshape(M, nb * 292)


def expected(orc, fmt, W, xq, M, N, K):
    y = orc.gemm_int(fmt & 255, W, xq, M, N, K)
    y32 = y.astype(np.float32)
    assert np.array_equal(y32.astype(np.float64), y), "case leaves the exact regime"
    return y32


def weights_dev(gq, fmt, W, N, K):
    w = to_dev(W)
    return gq.repack(fmt & 255, w, N, K) if fmt > 255 else w


def assert_bits(got, want, where):
    got = np.asarray(got, np.float32)
    same = got.view(np.uint32) == want.view(np.uint32)
    if not same.all():
        i = np.unravel_index(np.argmin(same), same.shape)
        raise AssertionError("%s: %d of %d outputs differ; first at %s: %r vs %r"
                             % (where, int((~same).sum()), same.size, i, got[i], want[i]))


def run_case(gq, orc, fmt, M, N, K, path, seed):
    rng = np.random.default_rng(seed)
    W, mag = exact_weights(rng, fmt, N, K)
    dx, qx = exact_acts(rng, M, K, mag)
    xq = q8K_bytes(dx, qx)
    want = expected(orc, fmt, W, xq, M, N, K)
    got = to_host(gq.gemm(fmt, weights_dev(gq, fmt, W, N, K), to_dev(xq), M, N, K, path=path))
    assert_bits(got, want, "fmt %d M=%d N=%d K=%d path %d" % (fmt, M, N, K, path))


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("M", [1, 3, 5, 8])
@pytest.mark.parametrize("N,K", [(37, 256), (130, 1024), (33, 4096), (9, 12288)])
def test_exact_gemv(dev, gq, orc, fmt, M, N, K):
    log("exact gemv fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    run_case(gq, orc, fmt, M, N, K, PATH_GEMV, seed=1000 + 7 * fmt + 131 * M + N + K)


@pytest.mark.parametrize("M", [1, 3, 16, 17, 40, 64])
@pytest.mark.parametrize("N,K", [(37, 256), (130, 4096), (48, 12288)])
def test_exact_small_m(dev, gq, orc, M, N, K):
    log("exact small-M M=%d N=%d K=%d" % (M, N, K))
    run_case(gq, orc, Q4, M, N, K, PATH_SKINNY, seed=2000 + 131 * M + N + K)


@pytest.mark.parametrize("fmt", [Q6, R + Q6])
@pytest.mark.parametrize("M", [1, 3, 8, 9, 16])
@pytest.mark.parametrize("N,K", [(37, 256), (70, 2304), (33, 4096), (40, 12288)])
def test_exact_small_m_q6K(dev, gq, orc, fmt, M, N, K):
    log("exact small-M q6_K fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    run_case(gq, orc, fmt, M, N, K, PATH_SKINNY, seed=2500 + fmt + 131 * M + N + K)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("M", [9, 70, 130])
@pytest.mark.parametrize("N,K", [(37, 256), (130, 1024), (200, 8192), (65, 12288)])
def test_exact_gemm(dev, gq, orc, fmt, M, N, K):
    log("exact gemm fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    run_case(gq, orc, fmt, M, N, K, PATH_GEMM, seed=3000 + 7 * fmt + 131 * M + N + K)


@pytest.mark.parametrize("fmt", [Q2, Q3, Q5, Q6, R + Q3, R + Q6])
def test_exact_gemm_128_row_tiles(dev, gq, orc, fmt):
    # 600 x 4160: the plane kernel's 128-row grid has 5 x 65 workgroups, more
    # than the 256 up to which it runs 64-row tiles (the cases above), so this
    # call takes the 128-row form (q6_K: still below the 2048 workgroups of
    # 128 x 128 from which its four-tile kernel runs); sampled rows across
    # every row tile, the ragged last one included
    M, N, K = 600, 4160, 512
    log("exact gemm 128-row tiles fmt=%d" % fmt)
    rng = np.random.default_rng(3500 + fmt)
    W, mag = exact_weights(rng, fmt, N, K)
    dx, qx = exact_acts(rng, M, K, mag)
    xq = q8K_bytes(dx, qx)
    got = to_host(gq.gemm(fmt, weights_dev(gq, fmt, W, N, K), to_dev(xq), M, N, K, path=PATH_GEMM))
    rows = np.array([0, 31, 32, 63, 64, 127, 128, 255, 256, 383, 384, 511, 512, 575, 599])
    want = orc.gemm_int(fmt & 255, W, xq, M, N, K, rows)
    w32 = want.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), want), "case leaves the exact regime"
    assert_bits(got[rows], w32, "fmt %d 128-row tiles" % fmt)


@pytest.mark.parametrize("fmt", [Q4, Q6, R + Q6, Q2])
@pytest.mark.parametrize("M", [1, 4, 40, 130])
def test_exact_group(dev, gq, orc, fmt, M):
    # three matrices in one launch, the automatic path
    log("exact group fmt=%d M=%d" % (fmt, M))
    rng = np.random.default_rng(4000 + fmt + M)
    K, Ns = 2048, [96, 40, 17]
    mats = [exact_weights(rng, fmt, N, K) for N in Ns]
    mag = np.concatenate([m for _, m in mats])
    dx, qx = exact_acts(rng, M, K, mag)
    xq = q8K_bytes(dx, qx)
    ws = [weights_dev(gq, fmt, W, N, K) for (W, _), N in zip(mats, Ns)]
    outs = gq.gemm_group(fmt, ws, to_dev(xq), M, Ns, K)
    for g, ((W, _), N) in enumerate(zip(mats, Ns)):
        assert_bits(to_host(outs[g]), expected(orc, fmt, W, xq, M, N, K),
                    "group fmt %d M=%d matrix %d" % (fmt, M, g))


@pytest.mark.parametrize("fmt", [Q4, Q6, Q5, Q3])
@pytest.mark.parametrize("M", [1, 4, 20, 100])
@pytest.mark.parametrize("K", [1024, 4096])
def test_exact_linear(dev, gq, orc, fmt, M, K):
    # the one-call layer from f32 activations (fused quantizer at decode shapes)
    log("exact linear fmt=%d M=%d K=%d" % (fmt, M, K))
    rng = np.random.default_rng(5000 + fmt + M + K)
    Ns = [64, 33]
    quiet = rng.integers(0, 256, K // 256)
    mats = [exact_weights(rng, fmt, N, K, quiet) for N in Ns]
    mag = np.concatenate([m for _, m in mats])
    dx, qx = exact_acts(rng, M, K, mag, spike=quiet)
    x = (qx * np.repeat(dx, 256, 1)).astype(np.float32)
    xq_want = q8K_bytes(dx, qx)
    assert np.array_equal(orc.quantize_q8K(x), xq_want)
    ws = [to_dev(W) for W, _ in mats]
    outs, xq = gq.linear_group(fmt, ws, to_dev(x), Ns)
    assert np.array_equal(to_host(xq), xq_want)
    for g, ((W, _), N) in enumerate(zip(mats, Ns)):
        assert_bits(to_host(outs[g]), expected(orc, fmt, W, xq_want, M, N, K),
                    "linear fmt %d M=%d K=%d matrix %d" % (fmt, M, K, g))
