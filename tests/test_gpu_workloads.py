"""Parity on the five Qwen3-shaped workloads at full size, in the launch
configuration the benchmark times (automatic path choice; consecutive matrices
that read one activation in one format form one group, and each group is one
gemmq_linear_group call: the activation quantized on the GPU with the matmul,
fused into one launch at decode shapes).  Rows of large M are sampled (8 seeded rows, always the
first and the last); the oracle computes those rows against every weight row.
Bit-exact q8_K bytes for the sampled rows; f32 outputs within
1e-5 * sum|w*xhat| + 1e-6.
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
    mid = rng.choice(np.arange(1, M - 1), size=6, replace=False)
    return np.array(sorted({0, M - 1, *mid.tolist()}))


def _launches(wl, max_group):
    """The benchmark's launches: runs of consecutive matrices with one input and
    one format, at most max_group long."""
    out = []
    for m in wl.matrices:
        if out and out[-1][-1].inp == m.inp and out[-1][-1].fmt == m.fmt and len(out[-1]) < max_group:
            out[-1].append(m)
        else:
            out.append([m])
    return out


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
        for ms in _launches(wl, gq.MAX_GROUP):
            m0 = ms[0]
            log("  M=%d launch %s" % (M, "+".join(m.name for m in ms)))
            Wd = [to_dev(g.weights[m.name]) for m in ms]
            if m0.inp not in xq_dev:  # the activation's first group quantizes it
                x = g.activations[(M, m0.inp)]
                ys, xq_dev[m0.inp] = gq.linear_group(m0.fmt, Wd, to_dev(x),
                                                     [m.N for m in ms])
                got = xq_dev[m0.inp][torch.as_tensor(rows, device="cuda:0")].cpu().numpy()
                want = orc.quantize_q8K(x[rows])
                assert np.array_equal(got, want), (name, M, m0.inp)
                xq_host[m0.inp] = want
            else:
                ys = gq.gemm_group(m0.fmt, Wd, xq_dev[m0.inp], M, [m.N for m in ms], m0.K)
            for mat, y in zip(ms, ys):
                W = g.weights[mat.name]
                yr = y[torch.as_tensor(rows, device="cuda:0")].cpu().numpy()
                yo = orc.gemm_int(mat.fmt, W, xq_host[mat.inp], len(rows), mat.N, mat.K)
                _, S = orc.gemm_dequant(mat.fmt, W, xq_host[mat.inp], len(rows), mat.N, mat.K)
                worst = assert_within(yr, yo, S, "%s M=%d %s" % (name, M, mat.name))
                log("    %s %dx%d fmt=%d worst |err|/S = %.3g"
                    % (mat.name, mat.N, mat.K, mat.fmt, worst))
            del Wd, ys
        del xq_dev
        torch.cuda.empty_cache()
