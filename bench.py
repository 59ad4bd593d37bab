#!/usr/bin/env python3
"""Benchmark of the packed linear layer (libgemmq) on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for each activation width K, quantize X to q8_K, then run every matrix of the
layer through the packed matmul.  The default workload is the Qwen3-8B-shaped
layer (q 4096x4096, k/v 1024x4096, o 4096x4096, gate/up 12288x4096, down
4096x12288, all q4_K; 108,527,616 weight bytes), run at M = 1 (decode GEMV,
weight GB/s), M = 512 (prefill GEMM, int8 TOP/s) and M = 8 (batched decode on
the small-M MFMA kernel, weight GB/s, reported as `batched_decode_m8`) and
M = 2048 (prefill, reported as `prefill_m2048`).

Each matrix reads the activation of its place in the layer (q/k/v the attention
input, o the attention output, gate/up the MLP input, down the MLP activation),
so a pass quantizes four activation tensors and runs seven matmuls.  Matrices
that read the same activation in the same format run as one group, and each
group is one gemmq_linear_group call: quantize its activation, then the packed
matmul (q/k/v, o, gate/up, down).  At M = 1 each call is one fused launch (every
GEMV workgroup quantizes the activation into its own LDS); at M = 512 it is a
quantizer launch and a GEMM launch.  --no-fuse calls gemmq_quantize_q8K and
gemmq_gemm_group separately; --no-group launches every matrix on its own.

Inputs are resident in HBM before timing starts.  So that the weights are
really streamed from HBM and not from the 256 MB last-level cache, the step
rotates over R copies of the layer's weights (R * 108.5 MB >= 1 GiB).  Passes
are submitted as eager launches on one stream; --graph instead captures one pass
per weight copy in a HIP graph and times the replays (slower on this stack).

Output: one JSON line.  `value` is the M=1 weight throughput of the whole step
(quantizer launches included); `secondary` the M=512 int8 throughput;
`roofline` / `roofline_m512` give the dominant kernels' algorithmic rate from
HIP events around batches of back-to-back launches against the MI355X peaks
(HBM 8 TB/s; dense int8 MFMA 5.0 POP/s) and against ceilings measured on the
same GPU (`ceilings`: a plain 1 GiB device copy, the library's int8 MFMA-only
loop with the shader clock it ran at, and the vendor library's plain int8 GEMM
at the largest matrix's shape); `cpu_baseline` times the CPU oracle
on a bounded sample, on all host cores and on one.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA, TOP/s
GIB = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="qwen3-8b-q4K")
    p.add_argument("--m", type=int, nargs="+", default=[1, 512, 8, 2048],
                   help="activation rows; the first is the headline (value), the second secondary")
    p.add_argument("--copies", type=int, default=0, help="rotating weight copies (0: auto, >=1 GiB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="time HIP-graph replays of each pass instead of eager launches")
    p.add_argument("--cpu-seconds", type=float, default=20.0)
    p.add_argument("--no-group", action="store_true",
                   help="one launch per matrix instead of grouping matrices that share an input")
    p.add_argument("--no-fuse", action="store_true",
                   help="separate quantizer and matmul calls instead of gemmq_linear_group")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="first run one plain device-to-device copy of MIB MiB (reference dispatch "
                        "for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


class Layer:
    """Device buffers for one workload: rotating weight copies, activations,
    q8_K buffers and outputs, all allocated before timing."""

    def __init__(self, wl, gen, Ms, copies, group=True, fuse=True):
        import torch

        import quant_packed_weight_amd as gq

        self.gq = gq
        self.wl = wl
        self.Ms = Ms
        self.fuse = fuse
        # launches: runs of consecutive matrices with one input and one format
        self.launches = []
        for m in wl.matrices:
            last = self.launches[-1] if self.launches else None
            if (group and last and last[-1].inp == m.inp and last[-1].fmt == m.fmt
                    and len(last) < gq.MAX_GROUP):
                last.append(m)
            else:
                self.launches.append([m])
        self.w = []
        base = {m.name: torch.from_numpy(gen.weights[m.name]).to("cuda:0") for m in wl.matrices}
        for r in range(copies):
            self.w.append({k: (v if r == 0 else v.clone()) for k, v in base.items()})
        self.x, self.xq, self.y = {}, {}, {}
        for M in Ms:
            for inp, K in wl.inputs():
                self.x[(M, inp)] = torch.from_numpy(gen.activations[(M, inp)]).to("cuda:0")
                self.xq[(M, inp)] = torch.empty(gq.q8K_bytes(M, K), dtype=torch.uint8,
                                                device="cuda:0")
            for m in wl.matrices:
                self.y[(M, m.name)] = torch.empty((M, m.N), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()

        # every launch's C arguments, built once: the timed loops only call the
        # library, so host-side Python stays well below the kernels' duration
        import ctypes

        P, I64 = ctypes.c_void_p, ctypes.c_int64
        self.lib = gq.lib()
        self.args = {}
        for M in Ms:
            for r in range(copies):
                for ms in self.launches:
                    n = len(ms)
                    m0 = ms[0]
                    wa = (P * n)(*[self.w[r][m.name].data_ptr() for m in ms])
                    ya = (P * n)(*[self.y[(M, m.name)].data_ptr() for m in ms])
                    na = (I64 * n)(*[m.N for m in ms])
                    self.args[(M, r, launch_name(ms))] = (
                        m0.fmt, n, wa, ya, na, self.xq[(M, m0.inp)].data_ptr(), M, m0.K,
                        gq.PATH_AUTO)
                    self.args[(M, r, launch_name(ms), "linear")] = (
                        m0.fmt, n, wa, ya, na, self.x[(M, m0.inp)].data_ptr(),
                        self.xq[(M, m0.inp)].data_ptr(), M, m0.K, gq.PATH_AUTO)
            for inp, K in wl.inputs():
                self.args[(M, "q", inp)] = (self.x[(M, inp)].data_ptr(),
                                            self.xq[(M, inp)].data_ptr(), M, K)

    def launch(self, ms, M, r, st):
        """Enqueue the matmul launch of the matrices `ms` (one input, one format)."""
        rc = self.lib.gemmq_gemm_group(*self.args[(M, r, launch_name(ms))], st)
        if rc:
            raise self.gq.GemmqError(rc, "gemm " + launch_name(ms))

    def linear(self, ms, M, r, st):
        """Enqueue quantize + matmul of the matrices `ms` in one library call."""
        rc = self.lib.gemmq_linear_group(*self.args[(M, r, launch_name(ms), "linear")], st)
        if rc:
            raise self.gq.GemmqError(rc, "linear " + launch_name(ms))

    def quantize(self, inp, K, M, st):
        rc = self.lib.gemmq_quantize_q8K(*self.args[(M, "q", inp)], st)
        if rc:
            raise self.gq.GemmqError(rc, "quantize")

    def run(self, M, r, stream):
        """Enqueue one pass at M rows on weight copy r."""
        st = stream.cuda_stream
        done = set()
        for ms in self.launches:
            inp = ms[0].inp
            if inp not in done:  # quantize each activation with its first use
                done.add(inp)
                if self.fuse:
                    self.linear(ms, M, r, st)
                    continue
                self.quantize(inp, ms[0].K, M, st)
            self.launch(ms, M, r, st)


def launch_name(ms):
    return "+".join(m.name for m in ms)


def time_passes(layer, M, steps, warmup, copies, stream):
    """Eager launches: seconds per pass."""
    import torch

    for s in range(warmup):
        layer.run(M, s % copies, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        layer.run(M, (warmup + s) % copies, stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def capture_graphs(layer, M, copies):
    """One HIP graph per weight copy, each holding one whole pass."""
    import torch

    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.run(M, 0, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.run(M, r, torch.cuda.current_stream())
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_graphs(graphs, steps, warmup):
    """Graph replays: seconds per pass."""
    import torch

    n = len(graphs)
    for s in range(warmup):
        graphs[s % n].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        graphs[(warmup + s) % n].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def fused_launch(M, K):
    """Whether gemmq_linear_group runs this shape as one fused quantize + GEMV
    launch: the library's rule (gemv.hip: rows of at most 16 blocks, M <= 4,
    M K/256 <= 32), restated here only to label the timings."""
    nb = K // 256
    return 1 <= M <= 4 and 1 <= nb <= 16 and M * nb <= 32


def kernel_rates(layer, M, steps, copies, stream):
    """Average duration of each matmul launch of the pass: two HIP events on the
    launch stream around a batch of back-to-back copies of that launch (weight
    copies rotated).  Where the pass runs a group as one fused quantize + GEMV
    launch, that launch is timed; otherwise the matmul launch alone, its
    activation quantized once beforehand."""
    import torch

    st = stream.cuda_stream
    for ms in layer.launches:
        layer.quantize(ms[0].inp, ms[0].K, M, st)
    per = {}
    n = max(steps, copies)
    for ms in layer.launches:
        fused = layer.fuse and fused_launch(M, ms[0].K)
        call = layer.linear if fused else layer.launch
        for r in range(copies):  # warm the launch path
            call(ms, M, r, st)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(n):
            call(ms, M, r % copies, st)
        e1.record(stream)
        torch.cuda.synchronize()
        per[launch_name(ms)] = (ms, e0.elapsed_time(e1) * 1e-3 / n, fused)
    return per


def profiled_traffic(fam, launches):
    """HBM bytes per launch of kernel family `fam` ("gemv" / "gemm") over the
    pass's launches, from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/traffic.json, FETCH scaled by the cold-copy factor).  None when
    the kernel sources changed since those counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)[fam]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for src in t.get("sources", []):
        with open(os.path.join(ROOT, "quant_packed_weight_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    per = t.get("per_launch", {})
    names = [launch_name(ms) for ms in launches]
    if h.hexdigest() != t.get("source_sha256") or any(n not in per for n in names):
        return None
    tot = sum(per[n]["read_bytes"] + per[n]["write_bytes"] for n in names)
    return round(tot / len(names))


def measured_ceilings(wl):
    """Ceilings measured on this GPU beside the datasheet peaks: a plain 1 GiB
    device-to-device copy (read + write bytes); the library's int8 MFMA-only
    loop (gemmq_probe_mfma_i8: independent accumulator chains, no memory
    traffic), with the shader clock it ran at from its in-kernel counters; and
    a plain int8 GEMM from the vendor library (torch._int_mm, int8 x int8 ->
    int32, no quantized format) at the largest matrix's shape with M = 512."""
    import torch

    import quant_packed_weight_amd as gq

    out = {}
    # MFMA-only loop: 2048 workgroups (8 per CU, two waves per SIMD), ~5 ms
    blocks, iters = 2048, 10000
    gq.probe_mfma_i8(100, blocks)
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _, clocks, nops = gq.probe_mfma_i8(iters, blocks)
        e1.record()
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) * 1e-3
        cyc, ticks = (int(v) for v in clocks.cpu())
        if best is None or dt < best[0]:
            best = (dt, nops, cyc, ticks)
    dt, nops, cyc, ticks = best
    out["mfma_i8_TOPs"] = round(nops / dt / 1e12, 1)
    out["mfma_i8_clock_GHz"] = round(cyc / ticks * 0.1, 3) if ticks > 0 else None
    n = GIB
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["copy_GBs"] = round(2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    big = max(wl.matrices, key=lambda m: m.N * m.K)
    try:
        a = torch.randint(-127, 128, (512, big.K), dtype=torch.int8, device="cuda:0")
        b = torch.randint(-127, 128, (big.K, big.N), dtype=torch.int8, device="cuda:0")
        for _ in range(3):
            torch._int_mm(a, b)
        e0.record()
        for _ in range(10):
            torch._int_mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        out["int8_gemm_TOPs"] = round(2 * 512 * big.N * big.K * 10 /
                                      (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        out["int8_gemm_shape"] = "512x%dx%d (torch._int_mm)" % (big.N, big.K)
    except Exception as e:  # not every build has an int8 GEMM
        out["int8_gemm_TOPs"] = None
        out["int8_gemm_error"] = type(e).__name__
    return out


def sample_rows(M, n=32, seed=512):
    """A seeded sample of n activation rows of M, the first and last included."""
    import numpy as np

    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, M - 1), size=min(n, M) - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], mid])).astype(np.int64)


def _oracle_rate(wl, gen, M1, M2, seconds, threads):
    """One bounded sample of the oracle with `threads` host threads: each matrix
    split into row ranges run concurrently (the C oracle releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    def run_all(pool, xq, M, rows=None):
        jobs = []
        for m in wl.matrices:
            W = gen.weights[m.name]
            step = -(-m.N // threads)
            for n0 in range(0, m.N, step):
                n1 = min(m.N, n0 + step)
                jobs.append(pool.submit(oracle.gemm_int, m.fmt, W[n0:n1], xq[m.inp], M, n1 - n0,
                                        m.K, rows))
        for j in jobs:
            j.result()

    res = {}
    with ThreadPoolExecutor(threads) as pool:
        passes, t0 = 0, time.perf_counter()
        while True:
            xq = {inp: oracle.quantize_q8K(gen.activations[(M1, inp)]) for inp, _ in wl.inputs()}
            run_all(pool, xq, M1)
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds or passes >= 2000:
                break
        res["m1"] = (passes, el)
        if M2:
            rows = sample_rows(M2)
            xq = {inp: oracle.quantize_q8K(gen.activations[(M2, inp)][rows])
                  for inp, _ in wl.inputs()}
            t0 = time.perf_counter()
            run_all(pool, xq, len(rows))
            res["m2"] = time.perf_counter() - t0
    return res


def cpu_baseline(wl, gen, M1, M2, seconds):
    """The oracle on a bounded sample of the same workload, on all of this host's
    cores (the row-parallel thin driver above) and on one core."""
    cores = len(os.sched_getaffinity(0))
    wbytes = sum(m.nbytes for m in wl.matrices)
    nrows = len(sample_rows(M2)) if M2 else 0
    ops2 = sum(2 * nrows * m.N * m.K for m in wl.matrices)
    out = {"kind": "oracle", "cores": cores}
    for label, threads in (("", cores), ("_1core", 1)):
        r = _oracle_rate(wl, gen, M1, M2, seconds / 4, threads)
        passes, el = r["m1"]
        out["value" + label] = wbytes * passes / el / 1e9
        if not label:
            out["unit"] = "GB/s"
            out["sample"] = ("%d full pass(es) of the %d-matrix layer at M=%d (quantize + "
                             "integer-route matmul, each matrix's rows split over %d threads), "
                             "%.1f s; the same with 1 thread in value_1core"
                             % (passes, len(wl.matrices), M1, threads, el))
        if M2:
            out["value_m%d%s" % (M2, label)] = ops2 / r["m2"] / 1e12
            if not label:
                out["unit_m%d" % M2] = "TOP/s"
                out["sample_m%d" % M2] = ("%d seeded rows of M=%d (first and last included) "
                                          "through all %d matrices, %.1f s (1 thread: value_m%d_1core)"
                                          % (nrows, M2, len(wl.matrices), r["m2"], M2))
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py: this build runs on exactly one GPU (the packed linear layer has no "
              "collective); --gpus %d is not supported" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import quant_packed_weight_amd as gq
    from quant_packed_weight_amd import synth

    assert torch.cuda.is_available(), "no GPU"
    gq.lib()
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[a.workload]
    Ms = [M for M in a.m]
    gen = synth.generate(a.workload, Ms=None if set(Ms) - set(wl.Ms) else set(Ms))
    if set(Ms) - set(wl.Ms):
        raise SystemExit("workload %s has M in %s" % (a.workload, wl.Ms))
    wbytes = sum(m.nbytes for m in wl.matrices)
    copies = a.copies or max(1, math.ceil(GIB / wbytes))
    layer = Layer(wl, gen, Ms, copies, group=not a.no_group, fuse=not a.no_fuse)
    stream = torch.cuda.current_stream()
    if a.copy_calibration:
        # a plain device copy of known size whose source is cold: after filling
        # it, 1 GiB of other writes pushes it out of L2 and the 256 MB MALL
        n = a.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        flush = torch.empty(GIB, dtype=torch.uint8, device="cuda:0")
        flush.fill_(7)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush

    t_eager = {M: time_passes(layer, M, a.steps, a.warmup, copies, stream) for M in Ms}
    rates = {M: kernel_rates(layer, M, a.steps, copies, stream) for M in Ms}
    if not a.graph:
        t = t_eager
    else:
        graphs = {M: capture_graphs(layer, M, copies) for M in Ms}
        t = {M: time_graphs(graphs[M], a.steps, a.warmup) for M in Ms}

    M1 = Ms[0]
    M2 = Ms[1] if len(Ms) > 1 else None
    ops = {M: sum(2 * M * m.N * m.K for m in wl.matrices) for M in Ms}

    def roof(M):
        per = rates[M]
        n_l = len(per)
        tot_t = sum(dt for _, dt, _ in per.values())
        fused = [k for k, (_, _, f) in per.items() if f]
        # the automatic path's kernel for the all-q4_K layer (the small-M kernel
        # at 17..64 rows on some launches only)
        kname = ("gemv_kernel" if M <= 2 else "skinny_q4k_kernel" if M <= 16
                 else "gemm_q4k_kernel")
        if fused:
            kname += " (quantizer fused into: %s)" % ", ".join(fused)
        if M <= 8:
            algo = sum(sum(m.nbytes for m in ms) for ms, _, _ in per.values())
            ach = algo / tot_t / 1e9
            return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": (profiled_traffic("gemv", layer.launches)
                                if a.workload == "qwen3-8b-q4K" and M == 1 else None),
                    "algo_bytes_per_launch": round(algo / n_l),
                    "kernel": kname, "launches_per_pass": n_l,
                    "avg_launch_us": round(tot_t / n_l * 1e6, 2),
                    "per_launch_GBs": {k: round(sum(m.nbytes for m in ms) / dt / 1e9, 1)
                                       for k, (ms, dt, _) in per.items()}}
        algo = sum(sum(2 * M * m.N * m.K for m in ms) for ms, _, _ in per.values())
        ach = algo / tot_t / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s", "frac": round(ach / INT8_PEAK_TOPS, 4),
                "traffic": (profiled_traffic("gemm", layer.launches)
                            if a.workload == "qwen3-8b-q4K" and M == 512 else None),
                "algo_ops_per_launch": round(algo / n_l),
                "kernel": kname, "launches_per_pass": n_l,
                "avg_launch_us": round(tot_t / n_l * 1e6, 2),
                "per_launch_TOPs": {k: round(sum(2 * M * m.N * m.K for m in ms) / dt / 1e12, 1)
                                    for k, (ms, dt, _) in per.items()}}

    value = wbytes / t[M1] / 1e9 if M1 <= 8 else ops[M1] / t[M1] / 1e12
    res = {
        "metric": "q4_K gemm_quant: weight GB/s at M=1 & int8 TOPS at M=512, % of roofline",
        "value": round(value, 1),
        "unit": "GB/s" if M1 <= 8 else "TOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(sum(t.values()) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": a.workload, "M": Ms, "matrices": len(wl.matrices),
                   "activations": len(wl.inputs()), "weight_bytes": wbytes,
                   "rotating_copies": copies, "submit": "hip_graph" if a.graph else "eager",
                   "calls": "separate quantize + matmul" if a.no_fuse else "gemmq_linear_group",
                   "launches": [launch_name(ms) for ms in layer.launches],
                   "ms_per_pass": {str(M): round(t[M] * 1e3, 4) for M in Ms},
                   "ms_per_pass_eager": {str(M): round(t_eager[M] * 1e3, 4) for M in Ms}},
        "roofline": roof(M1),
    }
    if M2:
        res["secondary"] = {"metric": "int8 TOP/s at M=%d" % M2,
                            "value": round(ops[M2] / t[M2] / 1e12, 1), "unit": "TOP/s"}
        res["roofline_m%d" % M2] = roof(M2)
    for M in Ms[2:]:
        # the rest of the M sweep: batched decode (weight GB/s) or prefill (int8 TOP/s)
        per = rates[M]
        rec = {"M": M, "us_per_pass": round(t[M] * 1e6, 2),
               "weight_GBs": round(wbytes / t[M] / 1e9, 1),
               "int8_TOPs": round(ops[M] / t[M] / 1e12, 2)}
        if M <= 16:
            rec["per_launch_GBs"] = {k: round(sum(m.nbytes for m in ms) / dt / 1e9, 1)
                                     for k, (ms, dt, _) in per.items()}
            res["batched_decode_m%d" % M] = rec
        else:
            rec["per_launch_TOPs"] = {k: round(sum(2 * M * m.N * m.K for m in ms) / dt / 1e12, 1)
                                      for k, (ms, dt, _) in per.items()}
            res["prefill_m%d" % M] = rec
    c = res["ceilings"] = measured_ceilings(wl)
    c["copy_frac_of_peak"] = round(c["copy_GBs"] / HBM_PEAK_GBS, 4)
    c["mfma_i8_frac_of_peak"] = round(c["mfma_i8_TOPs"] / INT8_PEAK_TOPS, 4)
    if c.get("int8_gemm_TOPs"):
        c["int8_gemm_frac_of_peak"] = round(c["int8_gemm_TOPs"] / INT8_PEAK_TOPS, 4)
    # the kernels against the measured ceilings as well as the datasheet peaks
    res["roofline"]["frac_of_measured_copy"] = round(res["roofline"]["achieved"] / c["copy_GBs"], 4)
    if M2:
        res["roofline_m%d" % M2]["frac_of_measured_mfma"] = round(
            res["roofline_m%d" % M2]["achieved"] / c["mfma_i8_TOPs"], 4)
    if M2 and c.get("int8_gemm_TOPs"):
        res["roofline_m%d" % M2]["vs_int8_gemm_library"] = round(
            res["roofline_m%d" % M2]["achieved"] / c["int8_gemm_TOPs"], 4)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, gen, M1, M2, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
