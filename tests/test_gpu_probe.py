"""GPU: the int8 MFMA ceiling loop (gemmq_probe_mfma_i8) that the benchmark
reads the GEMM against, the same loop with vector work beside every MFMA
(gemmq_probe_mfma_valu) and the read-only stream (gemmq_probe_read).

The loop's work is checked exactly, not just timed: summed over the 64 lanes of
a wave, the accumulators hold chains * iters * sum_{i,j} (A B)[i, j]
= chains * iters * sum_k (sum_i A[i, k]) (sum_j B[k, j]) whatever the output
layout, where lane l supplies row / column l % 32 and K values
16 (l // 32) .. 16 (l // 32) + 15 of the 32 x 32 x 32 int8 product (the operand
layout the GEMM kernels use).  Integer sums wrap modulo 2^32 like the device's.
"""
import numpy as np
import pytest

from gpu_util import device, log, to_host

pytestmark = pytest.mark.gpu


def operands(t):
    """The probe's per-thread operands as int8 bytes: four int32 words each."""
    a = np.array([t, 7 * t + 1, 13 * t + 2, 29 * t + 3], dtype=np.int64).astype(np.uint32)
    b = np.array([3 * t + 5, 11 * t + 7, 17 * t + 9, 23 * t + 11], dtype=np.int64).astype(np.uint32)
    return a.view(np.int8).astype(np.int64), b.view(np.int8).astype(np.int64)


def wave_sum(w, chains, iters):
    colA = np.zeros(32, dtype=np.int64)  # sum over rows i of A[i, k]
    rowB = np.zeros(32, dtype=np.int64)  # sum over columns j of B[k, j]
    for lane in range(64):
        a, b = operands(64 * w + lane)
        h = lane // 32
        colA[16 * h:16 * h + 16] += a
        rowB[16 * h:16 * h + 16] += b
    total = chains * iters * int((colA * rowB).sum())
    return np.int64(total).astype(np.uint64) & np.uint64(0xFFFFFFFF)


@pytest.mark.parametrize("iters,blocks", [(1, 1), (3, 5), (17, 300)])
def test_probe_work_is_exact(iters, blocks):
    device()
    import quant_packed_weight_amd as gq

    log("probe iters=%d blocks=%d" % (iters, blocks))
    out, clocks, ops = gq.probe_mfma_i8(iters, blocks)
    o = to_host(out).astype(np.int64).reshape(blocks, 4, 64)
    assert ops == 2 * 32768 * gq.PROBE_CHAINS * 4 * blocks * iters
    assert (o == o[0]).all(), "every workgroup computes the same sums"
    for w in range(4):
        got = np.uint64(int(o[0, w].sum()) & 0xFFFFFFFF)
        assert got == wave_sum(w, gq.PROBE_CHAINS, iters), (w, got)
    c = to_host(clocks)
    assert c[0] > 0 and c[1] >= 0


@pytest.mark.parametrize("valu", [0, 4, 8, 12, 16])
def test_probe_mfma_valu_work_is_exact(valu):
    # the loop with vector work beside the MFMAs (gemmq_probe_mfma_valu) does
    # the same matrix work on the same operands
    device()
    import quant_packed_weight_amd as gq

    iters, blocks = 9, 7
    log("probe mfma+valu valu=%d iters=%d blocks=%d" % (valu, iters, blocks))
    out, clocks, ops = gq.probe_mfma_valu(iters, blocks, valu)
    o = to_host(out).astype(np.int64).reshape(blocks, 4, 64)
    assert ops == 2 * 32768 * gq.PROBE_CHAINS * 4 * blocks * iters
    assert (o == o[0]).all()
    for w in range(4):
        got = np.uint64(int(o[0, w].sum()) & 0xFFFFFFFF)
        assert got == wave_sum(w, gq.PROBE_CHAINS, iters), (w, got)
    assert to_host(clocks)[0] > 0


def test_probe_clock_plausible():
    device()
    import quant_packed_weight_amd as gq

    out, clocks, ops = gq.probe_mfma_i8(20000, 64)
    cyc, ticks = (int(v) for v in to_host(clocks))
    assert ticks > 0
    ghz = cyc / ticks * 0.1
    log("probe shader clock %.3f GHz" % ghz)
    assert 0.3 < ghz < 3.5


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 10 * (1 << 20) + 16 * 7, 64 << 20])
def test_read_probe_reads_every_word_once(nbytes):
    # the XOR of every wave's fold is the XOR of every 32-bit word of the buffer
    # exactly when each 16-byte word is read once
    import torch

    import quant_packed_weight_amd as gq

    log("read probe %d bytes" % nbytes)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    out = gq.probe_read(src)
    torch.cuda.synchronize()
    folds = out.cpu().numpy().view(np.uint32)
    assert folds.size == gq.PROBE_READ_WORDS
    assert np.bitwise_xor.reduce(folds) == np.bitwise_xor.reduce(host)
