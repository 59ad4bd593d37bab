"""HIP-graph capture of the hot path (quantize + GEMV + GEMM), as the benchmark
submits it: every replay must equal the eager result bit for bit, with eager
work, synchronisations and changed inputs between the replays."""
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
    cases = [(gq.FMT_Q4K, 1, 640, 1024), (gq.FMT_Q6K, 1, 300, 768),
             (gq.FMT_Q4K, 40, 200, 512), (gq.FMT_Q6K, 130, 96, 1024)]
    bufs = []
    for fmt, M, N, K in cases:
        W = torch.from_numpy(synth.make_weights(rng, fmt, N, K)).cuda()
        X = torch.from_numpy(synth.make_activations(rng, M, K, True)).cuda()
        Xq = torch.empty(gq.q8K_bytes(M, K), dtype=torch.uint8, device="cuda")
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        bufs.append((fmt, M, N, K, W, X, Xq, Y))

    def run(stream):
        st = stream.cuda_stream
        for fmt, M, N, K, W, X, Xq, Y in bufs:
            assert gq.quantize_q8K_ptr(X.data_ptr(), Xq.data_ptr(), M, K, st) == 0
            assert gq.gemm_ptr(fmt, W.data_ptr(), Xq.data_ptr(), Y.data_ptr(), M, N, K,
                               gq.PATH_AUTO, st) == 0

    def eager_ref():
        run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return [(b[6].clone(), b[7].clone()) for b in bufs]

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
        for b in bufs:  # clobber outputs so a replay that skips work is caught
            b[6].fill_(0xAB)
            b[7].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (xq_ref, y_ref), b in zip(ref, bufs):
            assert torch.equal(b[6], xq_ref)
            assert torch.equal(b[7].view(torch.int32), y_ref.view(torch.int32))
        # eager work between replays, then new inputs: the next replay must follow them
        eager_ref()
        if rep == 1:
            for b in bufs:
                b[5].mul_(-0.5)
            ref = eager_ref()
