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


def _check_layer(orc, gq, name, wl, weights, acts, M):
    """Every launch of the layer at M rows through the automatic path, sampled rows
    against the oracle; acts maps an input name to its f32 activation."""
    import torch

    rows = _rows(M, wl.seed * 1000 + M)
    xq_dev = {}
    xq_host = {}
    for ms in _launches(wl, gq.MAX_GROUP):
        m0 = ms[0]
        log("  M=%d launch %s" % (M, "+".join(m.name for m in ms)))
        Wd = [to_dev(weights[m.name]) for m in ms]
        if m0.inp not in xq_dev:  # the activation's first group quantizes it
            x = acts[m0.inp]
            ys, xq_dev[m0.inp] = gq.linear_group(m0.fmt, Wd, to_dev(x),
                                                 [m.N for m in ms])
            got = xq_dev[m0.inp][torch.as_tensor(rows, device="cuda:0")].cpu().numpy()
            want = orc.quantize_q8K(x[rows])
            assert np.array_equal(got, want), (name, M, m0.inp)
            xq_host[m0.inp] = want
        else:
            ys = gq.gemm_group(m0.fmt, Wd, xq_dev[m0.inp], M, [m.N for m in ms], m0.K)
        for mat, y in zip(ms, ys):
            W = weights[mat.name]
            yr = y[torch.as_tensor(rows, device="cuda:0")].cpu().numpy()
            yo = orc.gemm_int(mat.fmt, W, xq_host[mat.inp], len(rows), mat.N, mat.K)
            _, S = orc.gemm_dequant(mat.fmt, W, xq_host[mat.inp], len(rows), mat.N, mat.K)
            worst = assert_within(yr, yo, S, "%s M=%d %s" % (name, M, mat.name))
            log("    %s %dx%d fmt=%d worst |err|/S = %.3g"
                % (mat.name, mat.N, mat.K, mat.fmt, worst))
        del Wd, ys
    del xq_dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload(dev, orc, name):
    import quant_packed_weight_amd as gq

    wl = synth.WORKLOADS[name]
    log("workload %s" % name)
    g = synth.generate(name)
    for M in wl.Ms:
        acts = {inp: g.activations[(M, inp)] for inp, _ in wl.inputs()}
        _check_layer(orc, gq, name, wl, g.weights, acts, M)


def test_qwen3_8b_mid_batch(dev, orc):
    # the Qwen3-8B q4_K layer at 17..64 rows, where the automatic choice mixes the
    # small-M kernel (q/k/v up to 48 rows, o and down up to 64) with the GEMM
    # (gate/up from 17 rows, q/k/v past 48); activations drawn for these M from
    # their own seed, in the workload's recipe
    import quant_packed_weight_amd as gq

    name = "qwen3-8b-q4K"
    wl = synth.WORKLOADS[name]
    g = synth.generate(name, Ms=set())
    for M in (24, 48, 64):
        log("workload %s M=%d" % (name, M))
        rng = np.random.default_rng(7000 + M)
        acts = {inp: synth.make_activations(rng, M, K, wl.outliers) for inp, K in wl.inputs()}
        _check_layer(orc, gq, name, wl, g.weights, acts, M)
