"""Parity on the five Qwen3-shaped workloads at full size, in the launch
configuration the benchmark times (automatic path choice, activations quantized
on the GPU).  Rows of large M are sampled (always the first and the last); the
oracle computes those rows against every weight row.  Bit-exact q8_K bytes for
the sampled rows; f32 outputs within 1e-5 * sum|w*xhat| + 1e-6.
"""
import numpy as np
import pytest

from gpu_util import assert_within, device, log, to_dev
from quant_packed_weight_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _rows(M, seed):
    if M <= 8:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, M - 1), size=2, replace=False)
    return np.array(sorted({0, M - 1, *mid.tolist()}))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload(dev, orc, name):
    import torch

    import quant_packed_weight_amd as gq

    wl = synth.WORKLOADS[name]
    log("workload %s" % name)
    g = synth.generate(name)
    for M in wl.Ms:
        rows = _rows(M, wl.seed * 1000 + M)
        xq_dev = {}
        xq_host = {}
        for inp, K in wl.inputs():
            x = g.activations[(M, inp)]
            xd = to_dev(x)
            xq_dev[inp] = gq.quantize_q8K(xd)
            got = xq_dev[inp][torch.as_tensor(rows, device="cuda:0")].cpu().numpy()
            want = orc.quantize_q8K(x[rows])
            assert np.array_equal(got, want), (name, M, inp)
            xq_host[inp] = want
            del xd
        for mat in wl.matrices:
            log("  M=%d %s %dx%d fmt=%d" % (M, mat.name, mat.N, mat.K, mat.fmt))
            W = g.weights[mat.name]
            Wd = to_dev(W)
            y = gq.gemm(mat.fmt, Wd, xq_dev[mat.inp], M, mat.N, mat.K)
            ys = y[torch.as_tensor(rows, device="cuda:0")].cpu().numpy()
            yo = orc.gemm_int(mat.fmt, W, xq_host[mat.inp], len(rows), mat.N, mat.K)
            _, S = orc.gemm_dequant(mat.fmt, W, xq_host[mat.inp], len(rows), mat.N, mat.K)
            worst = assert_within(ys, yo, S, "%s M=%d %s" % (name, M, mat.name))
            log("    worst |err|/S = %.3g" % worst)
            del Wd, y
        del xq_dev
        torch.cuda.empty_cache()
