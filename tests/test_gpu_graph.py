"""HIP-graph capture of the hot path (quantize + GEMV + small-M MFMA + GEMM,
single and grouped launches, gemmq_linear_group: the fused quantize + GEMV launch and its
two-launch form, and gemmq_linear_silu_mul on its fused, GEMV and GEMM routes), as the benchmark submits it: every replay must equal the eager result
bit for bit, with eager work, synchronisations and changed inputs between the
replays."""
import numpy as np
import pytest

from gpu_util import device, log

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch

    import quant_packed_weight_amd as gq
    from quant_packed_weight_amd import synth

    device()
    rng = np.random.default_rng(99)
    # every format, and the repacked layouts (repacked once, before capture)
    cases = [(gq.FMT_Q4K, 1, 640, 1024), (gq.FMT_Q6K, 1, 300, 768),
             (gq.FMT_Q4K, 40, 200, 512), (gq.FMT_Q6K, 130, 96, 1024),
             (gq.FMT_Q2K, 1, 100, 2048), (gq.FMT_Q3K, 3, 70, 512), (gq.FMT_Q5K, 1, 129, 4096),
             (gq.FMT_Q2K, 33, 64, 512), (gq.FMT_Q3K, 40, 65, 1024), (gq.FMT_Q5K, 64, 100, 768),
             (gq.FMT_Q6K_R, 1, 200, 3072), (gq.FMT_Q3K_R, 50, 90, 1024),
             (gq.FMT_Q4K, 80, 96, 512),  # q4_K GEMM
             (gq.FMT_Q4K, 8, 333, 4096), (gq.FMT_Q4K, 27, 70, 12288)]  # small-M MFMA kernel
    bufs = []
    for fmt, M, N, K in cases:
        W = torch.from_numpy(synth.make_weights(rng, fmt & 255, N, K)).cuda()
        if fmt > 255:
            W = gq.repack(fmt & 255, W, N, K)
        X = torch.from_numpy(synth.make_activations(rng, M, K, True)).cuda()
        Xq = torch.empty(gq.q8K_bytes(M, K), dtype=torch.uint8, device="cuda")
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        bufs.append((fmt, M, N, K, W, X, Xq, Y))

    # grouped launches: two matrices sharing one input, GEMV and GEMM
    groups = []
    for M in (1, 12, 40, 70):
        K, Ns = 1024, (300, 77)
        Ws = [torch.from_numpy(synth.make_weights(rng, gq.FMT_Q4K, N, K)).cuda() for N in Ns]
        X = torch.from_numpy(synth.make_activations(rng, M, K, True)).cuda()
        Xq = torch.empty(gq.q8K_bytes(M, K), dtype=torch.uint8, device="cuda")
        Ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for N in Ns]
        groups.append((M, K, Ns, Ws, X, Xq, Ys))

    # gemmq_linear_group: fused at (M 1, K 4096) and (M 2, K 1024), two launches
    # at (M 1, K 12288), (M 40, K 1024: small-M MFMA), (M 70: GEMM)
    linears = []
    for M, K in ((1, 4096), (2, 1024), (1, 12288), (40, 1024), (8, 4096), (70, 1024)):
        Ns = (260, 33)
        Ws = [torch.from_numpy(synth.make_weights(rng, gq.FMT_Q4K, N, K)).cuda() for N in Ns]
        X = torch.from_numpy(synth.make_activations(rng, M, K, True)).cuda()
        Xq = torch.empty(gq.q8K_bytes(M, K), dtype=torch.uint8, device="cuda")
        Ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for N in Ns]
        linears.append((M, K, Ns, Ws, X, Xq, Ys))

    # gemmq_linear_silu_mul: fused (M 1, K 2048), plain GEMV (M 1, K 8192), GEMM
    # (M 70), small-M MFMA (M 40 and 20)
    silus = []
    for fmt, M, K, N in ((gq.FMT_Q4K, 1, 2048, 300), (gq.FMT_Q6K, 1, 8192, 129),
                         (gq.FMT_Q4K, 70, 1024, 200), (gq.FMT_Q4K, 40, 1024, 200),
                         (gq.FMT_Q4K, 20, 3072, 90)):
        Wg = torch.from_numpy(synth.make_weights(rng, fmt, N, K)).cuda()
        Wu = torch.from_numpy(synth.make_weights(rng, fmt, N, K)).cuda()
        X = torch.from_numpy(synth.make_activations(rng, M, K, True)).cuda()
        Xq = torch.empty(gq.q8K_bytes(M, K), dtype=torch.uint8, device="cuda")
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        silus.append((fmt, M, N, K, Wg, Wu, X, Xq, Y))

    def run(stream):
        st = stream.cuda_stream
        for fmt, M, N, K, W, X, Xq, Y in bufs:
            assert gq.quantize_q8K_ptr(X.data_ptr(), Xq.data_ptr(), M, K, st) == 0
            assert gq.gemm_ptr(fmt, W.data_ptr(), Xq.data_ptr(), Y.data_ptr(), M, N, K,
                               gq.PATH_AUTO, st) == 0
        for M, K, Ns, Ws, X, Xq, Ys in groups:
            assert gq.quantize_q8K_ptr(X.data_ptr(), Xq.data_ptr(), M, K, st) == 0
            assert gq.gemm_group_ptr(gq.FMT_Q4K, [w.data_ptr() for w in Ws],
                                     [y.data_ptr() for y in Ys], list(Ns), Xq.data_ptr(), M, K,
                                     gq.PATH_AUTO, st) == 0
        for M, K, Ns, Ws, X, Xq, Ys in linears:
            assert gq.linear_group_ptr(gq.FMT_Q4K, [w.data_ptr() for w in Ws],
                                       [y.data_ptr() for y in Ys], list(Ns), X.data_ptr(),
                                       Xq.data_ptr(), M, K, gq.PATH_AUTO, st) == 0
        for fmt, M, N, K, Wg, Wu, X, Xq, Y in silus:
            assert gq.lib().gemmq_linear_silu_mul(fmt, Wg.data_ptr(), Wu.data_ptr(), X.data_ptr(),
                                                  Xq.data_ptr(), Y.data_ptr(), M, N, K,
                                                  gq.PATH_AUTO, st) == 0

    def outputs():
        out = [(b[6], b[7]) for b in bufs]
        for M, K, Ns, Ws, X, Xq, Ys in groups + linears:
            out += [(Xq, y) for y in Ys]
        out += [(b[7], b[8]) for b in silus]
        return out

    def eager_ref():
        run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return [(xq.clone(), y.clone()) for xq, y in outputs()]

    ref = eager_ref()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(4):
        log("replay %d" % rep)
        for xq, y in outputs():  # clobber outputs so a replay that skips work is caught
            xq.fill_(0xAB)
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (xq_ref, y_ref), (xq, y) in zip(ref, outputs()):
            assert torch.equal(xq, xq_ref)
            assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
        # eager work between replays, then new inputs: the next replay must follow them
        eager_ref()
        if rep == 1:
            for b in bufs:
                b[5].mul_(-0.5)
            for grp in groups:
                grp[4].mul_(-0.5)
            for b in silus:
                b[6].mul_(-0.5)
            ref = eager_ref()
