"""Pins of the oracle's load-time repack (CPU only).

The repack is a byte permutation with a closed form: the blocks' fields, each
stored for all blocks in block order.  Checked against numpy slicing of the
block array (a different construction from the oracle's copy loop), for the
field alignment it exists for, as a permutation (nothing lost or duplicated),
and on the refusal of formats without a repacked layout.
"""
import numpy as np
import pytest

from quant_packed_weight_amd import synth

FIELDS = {14: (128, 64, 16, 2), 11: (32, 64, 12, 2)}


@pytest.mark.parametrize("fmt", [11, 14])
@pytest.mark.parametrize("N,K", [(1, 256), (3, 768), (17, 4096), (64, 1024)])
def test_repack_closed_form(orc, fmt, N, K):
    rng = np.random.default_rng(N + K + fmt)
    W = synth.make_weights(rng, fmt, N, K)
    got = orc.repack(fmt, W, N, K)
    assert got.shape == W.shape
    blocks = W.reshape(-1, sum(FIELDS[fmt]))
    parts, off = [], 0
    for f in FIELDS[fmt]:
        parts.append(blocks[:, off:off + f].reshape(-1))
        off += f
    assert np.array_equal(got.reshape(-1), np.concatenate(parts))


@pytest.mark.parametrize("fmt", [11, 14])
def test_repack_is_a_permutation_with_aligned_fields(orc, fmt):
    N, K = 5, 2560
    nb = N * K // 256
    # every byte distinct by position: tag each byte with its (block, offset)
    bb = sum(FIELDS[fmt])
    idx = np.arange(nb * bb, dtype=np.int64)
    W = (idx % 251).astype(np.uint8)
    got = orc.repack(fmt, W, N, K).reshape(-1)
    assert np.array_equal(np.sort(got), np.sort(W))
    # field k of block i starts at sum_{j<k} nb*f_j + i*f_k: 16-byte aligned for
    # every field of 16+ bytes per block (the others are 2- and 4-byte fields)
    start = 0
    for f in FIELDS[fmt]:
        for i in (0, 1, nb - 1):
            s = start + i * f
            assert s % 16 == 0 or f < 16
            src = i * bb + (sum(FIELDS[fmt][:FIELDS[fmt].index(f)]))
            assert np.array_equal(got[s:s + f], W[src:src + f])
        start += nb * f


def test_repack_refuses_other_formats(orc):
    for fmt in (10, 12, 13):
        with pytest.raises(ValueError):
            orc.repack(fmt, synth.make_weights(np.random.default_rng(0), fmt, 2, 256), 2, 256)
