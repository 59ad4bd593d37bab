"""Helpers for the GPU parity tests (the oracle side of every comparison runs on
the host CPU; the device side goes through libgemmq's C ABI)."""
from __future__ import annotations

import sys

import numpy as np

TOL_REL = 1e-5  # the pages' scaled relative bound for reordered f32 sums
TOL_ABS = 1e-6


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    import torch

    import quant_packed_weight_amd as gq

    assert torch.cuda.is_available(), "no GPU visible"
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), arch
    gq.lib()  # raises if the library is not built
    return torch.device("cuda:0")


def to_dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def to_host(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_within(y, y_ref, S, where=""):
    """|y - y_ref| <= 1e-5 * S + 1e-6 element by element."""
    y = np.asarray(y, dtype=np.float64)
    assert y.shape == y_ref.shape == S.shape, (y.shape, y_ref.shape, S.shape)
    assert np.all(np.isfinite(y)), where + ": non-finite output"
    err = np.abs(y - y_ref)
    bound = TOL_REL * S + TOL_ABS
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s: y=%r ref=%r S=%r"
                             % (where, int(bad.sum()), bad.size, i, y[i], y_ref[i], S[i]))
    return float((err / np.maximum(S, 1e-30)).max()) if err.size else 0.0
