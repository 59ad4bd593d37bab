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
(quantizer launches included); `secondary` the M=512 int8 throughput, with the
matmul kernels' own rate beside it; `roofline` / `roofline_m512` give the
dominant kernels' algorithmic rate against the MI355X peaks (HBM 8 TB/s; dense
int8 MFMA 5.0 POP/s), each launch timed by HIP events on its stream around a
batch of back-to-back copies of it that rotate over >= 1 GiB of weights, and,
where the committed rocprofv3 runs of this benchmark still match the kernel
sources, the same launches' kernel-trace durations and HBM bytes
(profiles/kernel_profile.json); `quantizer` times the standalone q8_K
quantizer at the prefill widths; `ceilings` are measured on the same GPU: the
library's read-only stream over 2 GiB, a plain 1 GiB device copy, the
library's int8 MFMA-only loop with the shader clock it ran at, and the vendor
library's plain int8 GEMM at the largest matrix's shape.  `cpu_baseline` times
the CPU oracle on a bounded sample: the benchmarked workload on the physical
cores this process may use and on one, the other workloads of the set on one,
and the oracle quantizer alone on 512 x 1024.
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
NUM_CUS = 256              # MI355X compute units (4 SIMDs each)


def progress(msg):
    """A progress line on stderr (the JSON result is the only line on stdout)."""
    print("bench: " + msg, file=sys.stderr, flush=True)


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
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip the short timing of the set's other workloads")
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
        self.rot = {}  # per-launch rotating weight copies (launch_weights)
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


def fused_launch(M, K, rows):
    """Whether gemmq_linear_group runs this shape as one fused quantize + GEMV
    launch: the library's rule (gemv.hip: rows of at most 16 blocks, M <= 4,
    M K/256 <= 32, and rows x M x K/256 below 2^19, or below 2^18 where each
    wave would quantize four blocks -- larger calls quantize in a launch of their
    own), restated here only to label the timings."""
    nb = K // 256
    if not (1 <= M <= 4 and 1 <= nb <= 16 and M * nb <= 32):
        return False
    work = rows * M * nb
    mt = 1 if M <= 1 else 2 if M <= 2 else 4
    p = {1: 16, 2: 8, 4: 4, 8: 2}.get(nb, 1)
    qb = min(4, -(-mt * (16 // p if p > 1 else 16) // 8))
    return work < (1 << 19) and not (qb >= 4 and work >= (1 << 18))


def launch_weights(layer, ms, copies):
    """Weight copies that one launch rotates through when it is timed on its
    own: the layer's copies, then clones of this launch's matrices until the
    copies hold at least 1 GiB, so that every launch of the batch streams its
    weights from HBM (a small launch cycling through the layer's copies alone
    would find them in the 256 MB last-level cache)."""
    n = sum(m.nbytes for m in ms)
    want = max(copies, math.ceil(GIB / max(n, 1)))
    ws = [layer.w[r] for r in range(copies)]
    for _ in range(copies, want):
        ws.append({m.name: layer.w[0][m.name].clone() for m in ms})
    return ws


def kernel_rates(layer, M, steps, copies, stream):
    """Average duration of each matmul launch of the pass: two HIP events on the
    launch stream around a batch of back-to-back copies of that launch, rotating
    over at least 1 GiB of weight copies (launch_weights).  Where the pass runs
    a group as one fused quantize + GEMV launch, that launch is timed; otherwise
    the matmul launch alone, its activation quantized once beforehand."""
    import ctypes

    import torch

    P, I64 = ctypes.c_void_p, ctypes.c_int64
    st = stream.cuda_stream
    lib = layer.lib
    for ms in layer.launches:
        layer.quantize(ms[0].inp, ms[0].K, M, st)
    per = {}
    for ms in layer.launches:
        key = launch_name(ms)
        if key not in layer.rot:
            layer.rot[key] = launch_weights(layer, ms, copies)
        ws = layer.rot[key]
        fused = layer.fuse and fused_launch(M, ms[0].K, sum(m.N for m in ms))
        n = len(ms)
        m0 = ms[0]
        ya = (P * n)(*[layer.y[(M, m.name)].data_ptr() for m in ms])
        na = (I64 * n)(*[m.N for m in ms])
        xq = layer.xq[(M, m0.inp)].data_ptr()
        calls = []
        for w in ws:
            wa = (P * n)(*[w[m.name].data_ptr() for m in ms])
            if fused:
                calls.append((lib.gemmq_linear_group,
                              (m0.fmt, n, wa, ya, na, layer.x[(M, m0.inp)].data_ptr(), xq, M,
                               m0.K, layer.gq.PATH_AUTO, st)))
            else:
                calls.append((lib.gemmq_gemm_group,
                              (m0.fmt, n, wa, ya, na, xq, M, m0.K, layer.gq.PATH_AUTO, st)))
        reps = max(steps, len(calls))
        for f, args in calls[:3]:  # warm the launch path
            if f(*args):
                raise layer.gq.GemmqError(-1, key)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            f, args = calls[i % len(calls)]
            rc = f(*args)
            if rc:
                raise layer.gq.GemmqError(rc, key)
        e1.record(stream)
        torch.cuda.synchronize()
        per[key] = (ms, e0.elapsed_time(e1) * 1e-3 / reps, fused)
    return per


def quantizer_rates(layer, M, steps, stream):
    """Average duration of the standalone q8_K quantizer launch for each
    activation of the pass at M rows, timed like kernel_rates over at least
    1 GiB of rotating activation copies (so the f32 input streams from HBM).
    Algorithmic bytes: the f32 input read plus the q8_K output written."""
    import torch

    st = stream.cuda_stream
    out = {}
    for inp, K in layer.wl.inputs():
        x = layer.x[(M, inp)]
        xq = layer.xq[(M, inp)]
        nbytes = M * K * 4 + layer.gq.q8K_bytes(M, K)
        nx = max(1, math.ceil(GIB / (M * K * 4)))
        xs = [x] + [x.clone() for _ in range(nx - 1)]
        reps = max(steps, nx)
        for i in range(3):  # warm the launch path
            layer.lib.gemmq_quantize_q8K(xs[i % nx].data_ptr(), xq.data_ptr(), M, K, st)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            rc = layer.lib.gemmq_quantize_q8K(xs[i % nx].data_ptr(), xq.data_ptr(), M, K, st)
            if rc:
                raise layer.gq.GemmqError(rc, "quantize " + inp)
        e1.record(stream)
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) * 1e-3 / reps
        del xs
        out["%s %dx%d" % (inp, M, K)] = {
            "us": round(dt * 1e6, 2), "algo_bytes": nbytes,
            "GBs": round(nbytes / dt / 1e9, 1), "frac": round(nbytes / dt / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def profiled(workload, M, launches):
    """Per-launch figures of this workload at M rows from the committed
    rocprofv3 runs of this benchmark (profiles/kernel_profile.json): the
    kernel-trace average duration (us) and, when the counter runs were taken,
    the HBM bytes read and written (FETCH_SIZE scaled by a cold device copy's
    reading, WRITE_SIZE), per launch.  None when the sources of the kernels
    profiled changed since, or the runs do not cover these launches."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "kernel_profile.json")
    try:
        with open(path) as f:
            t = json.load(f)
        rec = t["runs"]["%s M=%d" % (workload, M)]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for src in rec.get("sources", []):
        try:
            with open(os.path.join(ROOT, "quant_packed_weight_amd", "csrc", src), "rb") as f:
                h.update(f.read())
        except OSError:
            return None
    per = rec.get("per_launch", {})
    names = [launch_name(ms) for ms in launches]
    if h.hexdigest() != rec.get("source_sha256") or any(n not in per for n in names):
        return None
    return {"per_launch": {n: per[n] for n in names}, "summary": rec.get("summary")}


def kernel_label(M):
    """The kernel the automatic path runs for an all-q4_K layer at M rows (the
    library's path choice, restated here only to label the record)."""
    if M <= 2:
        return "gemv_kernel"
    if M <= 64:
        return "skinny_q4k_kernel"
    return "gemm_q4k4_kernel" if M >= 1024 else "gemm_q4k2_kernel"


def measured_ceilings(wl, sizes=None):
    """Ceilings measured on this GPU beside the datasheet peaks: the library's
    read-only stream over 2 GiB (gemmq_probe_read, the GEMV's bound: it only
    reads weights); a plain 1 GiB device-to-device copy (read + write bytes);
    the library's int8 MFMA-only
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
    # the same loop with v independent f32 FMAs after every MFMA
    # (gemmq_probe_mfma_valu), two waves per SIMD as the GEMMs run: shader
    # clocks per MFMA and SIMD against v, and what a vector instruction costs
    # once the MFMA no longer hides it
    blocks_v, iters_v = 2 * NUM_CUS, 4000
    per = {}
    for v in (0, 4, 8, 12, 16):
        gq.probe_mfma_valu(10, blocks_v, v)
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            _, clocks, _ = gq.probe_mfma_valu(iters_v, blocks_v, v)
            e1.record()
            torch.cuda.synchronize()
            dt_v = e0.elapsed_time(e1) * 1e-3
            cyc_v, ticks_v = (int(x) for x in clocks.cpu())
            if best is None or dt_v < best[0]:
                best = (dt_v, cyc_v, ticks_v)
        dt_v, cyc_v, ticks_v = best
        ghz = cyc_v / ticks_v * 0.1 if ticks_v > 0 else out["mfma_i8_clock_GHz"]
        mfma_per_simd = blocks_v * 4 * iters_v * gq.PROBE_CHAINS / (4 * NUM_CUS)
        per[str(v)] = round(dt_v * ghz * 1e9 / mfma_per_simd, 1)
    out["mfma_valu_clk_per_mfma"] = per
    out["mfma_valu_note"] = ("shader clocks per int8 32x32x32 MFMA and SIMD with v independent "
                             "f32 FMAs after each, two waves per SIMD (gemmq_probe_mfma_valu)")
    out["valu_clk_per_instr"] = round((per["16"] - per["8"]) / 8, 2)
    # read-only stream (gemmq_probe_read) over 2 GiB: each launch reads more
    # than the last-level cache holds, so every byte comes from HBM
    n = 2 * GIB
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    gq.probe_read(src)
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gq.probe_read(src)
        e1.record()
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) * 1e-3
        best = dt if best is None else min(best, dt)
    out["read_GBs"] = round(n / best / 1e9, 1)
    # the same stream over as many bytes as each launch's weights, rotating
    # over slices of the 2 GiB buffer (cold): what a plain read of those bytes
    # takes, fixed launch costs included
    same = {}
    lib = gq.lib()
    fold = torch.empty(gq.PROBE_READ_WORDS, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    for name, nbytes in (sizes or {}).items():
        # the C call with its arguments built beforehand, as the matmul launches
        # are timed (the Python wrapper's own cost would exceed the kernel's)
        al = -(-nbytes // 256) * 256
        nb16 = nbytes - nbytes % 16
        ptrs = [src.data_ptr() + o for o in range(0, n - al + 1, al)]
        reps = max(50, len(ptrs))
        for p in ptrs[:3]:
            lib.gemmq_probe_read(p, nb16, fold.data_ptr(), st)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            if lib.gemmq_probe_read(ptrs[i % len(ptrs)], nb16, fold.data_ptr(), st):
                raise gq.GemmqError(-1, "gemmq_probe_read")
        e1.record()
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) * 1e-3 / reps
        same[name] = {"bytes": nbytes, "us": round(dt * 1e6, 3), "GBs": round(nbytes / dt / 1e9, 1)}
    if same:
        out["read_same_bytes"] = same
    # the same launch on 16 bytes: what any launch of the pass costs at the least
    # (dispatch, one wave's load round trip, completion), timed back to back
    for p in [src.data_ptr()] * 3:
        lib.gemmq_probe_read(p, 16, fold.data_ptr(), st)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(200):
        lib.gemmq_probe_read(src.data_ptr(), 16, fold.data_ptr(), st)
    e1.record()
    torch.cuda.synchronize()
    out["launch_floor_us"] = round(e0.elapsed_time(e1) * 1e3 / 200, 3)
    del src
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


def other_workloads(main_name, steps, warmup):
    """The set's other workloads (a single q4_K matrix at M = 8, the Qwen3-0.6B
    layer at M = 1 and 512, the Qwen3-1.7B layer with its q6_K head at M = 1
    and 512), each pass timed as the main workload's (eager launches over
    >= 1 GiB of rotating weight copies): microseconds per pass, weight GB/s and
    int8 TOP/s, and the path each launch takes."""
    import torch

    from quant_packed_weight_amd import synth

    out = {}
    for name, wl in synth.WORKLOADS.items():
        if name == main_name:
            continue
        gen = synth.generate(name)
        wbytes = sum(m.nbytes for m in wl.matrices)
        copies = max(1, math.ceil(GIB / wbytes))
        layer = Layer(wl, gen, list(wl.Ms), copies)
        stream = torch.cuda.current_stream()
        rec = {"weight_bytes": wbytes, "launches": [launch_name(ms) for ms in layer.launches]}
        for M in wl.Ms:
            t = time_passes(layer, M, steps, warmup, copies, stream)
            ops = sum(2 * M * m.N * m.K for m in wl.matrices)
            rec["M=%d" % M] = {"us_per_pass": round(t * 1e6, 2),
                               "weight_GBs": round(wbytes / t / 1e9, 1),
                               "int8_TOPs": round(ops / t / 1e12, 2)}
        out[name] = rec
        del layer, gen
        torch.cuda.empty_cache()
        progress("%s timed" % name)
    return out


def host_cores():
    """Logical CPUs of the host, those this process may run on, and the
    physical cores behind the latter (from the sysfs CPU topology)."""
    aff = sorted(os.sched_getaffinity(0))
    phys = set()
    for c in aff:
        base = "/sys/devices/system/cpu/cpu%d/topology/" % c
        try:
            with open(base + "physical_package_id") as f:
                pkg = f.read().strip()
            with open(base + "core_id") as f:
                core = f.read().strip()
            phys.add((pkg, core))
        except OSError:
            phys.add(("?", str(c)))
    return {"host_logical_cpus": os.cpu_count(), "affinity_logical_cpus": len(aff),
            "affinity_physical_cores": len(phys)}


def _oracle_workload(name, seconds, rows_cap):
    """One core: one of the benchmark's workloads through the oracle (quantize +
    integer-route matmul of every matrix), whole passes repeated for about
    `seconds`, or for M > 64 a seeded sample of at most `rows_cap` rows
    (first and last included), extrapolated per multiply-accumulate."""
    import numpy as np

    import oracle
    from quant_packed_weight_amd import synth

    g = synth.generate(name)
    wl = g.workload
    out = {}
    for M in wl.Ms:
        rows = sample_rows(M, rows_cap) if M > 64 else None
        nr = M if rows is None else len(rows)
        passes, t0 = 0, time.perf_counter()
        while True:
            for inp, _ in wl.inputs():
                x = g.activations[(M, inp)]
                xq = oracle.quantize_q8K(x if rows is None else np.ascontiguousarray(x[rows]))
                for m in wl.matrices:
                    if m.inp == inp:
                        oracle.gemm_int(m.fmt, g.weights[m.name], xq, nr, m.N, m.K)
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds or rows is not None:
                break
        mac = sum(nr * m.N * m.K for m in wl.matrices)
        wb = sum(m.nbytes for m in wl.matrices)
        rec = {"seconds": round(el, 3), "passes": passes, "GMACs": round(mac * passes / el / 1e9, 3)}
        if rows is None:
            rec["us_per_pass"] = round(el / passes * 1e6, 1)
            rec["weight_GBs"] = round(wb * passes / el / 1e9, 4)
        else:
            full = sum(M * m.N * m.K for m in wl.matrices)
            rec["sample"] = "%d of %d rows, extrapolated per MAC" % (nr, M)
            rec["ms_per_pass_extrapolated"] = round(el * full / mac * 1e3, 1)
        out["M=%d" % M] = rec
    del g
    return out


def _oracle_quantizer(M, K, seconds, threads):
    """The oracle's q8_K quantizer on an M x K f32 activation, rows split over
    `threads` host threads (the C call releases the GIL): microseconds per call."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    x = np.random.default_rng(512).standard_normal((M, K), dtype=np.float32)
    step = -(-M // threads)
    parts = [np.ascontiguousarray(x[r:r + step]) for r in range(0, M, step)]
    with ThreadPoolExecutor(threads) as pool:
        list(pool.map(oracle.quantize_q8K, parts))
        n, t0 = 0, time.perf_counter()
        while True:
            list(pool.map(oracle.quantize_q8K, parts))
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return el / n * 1e6


def cpu_baseline(wl, gen, M1, M2, seconds):
    """The oracle on a bounded sample of the benchmarked workload, on the
    physical cores this process may use (the row-parallel thin driver above)
    and on one core; the other workloads of the set on one core; and the
    oracle's quantizer alone on a 512 x 1024 activation."""
    hc = host_cores()
    cores = max(1, hc["affinity_physical_cores"])
    wbytes = sum(m.nbytes for m in wl.matrices)
    nrows = len(sample_rows(M2)) if M2 else 0
    ops2 = sum(2 * nrows * m.N * m.K for m in wl.matrices)
    out = {"kind": "oracle", "cores": cores}
    out.update(hc)
    for label, threads in (("", cores), ("_1core", 1)):
        r = _oracle_rate(wl, gen, M1, M2, seconds / 4, threads)
        passes, el = r["m1"]
        out["value" + label] = wbytes * passes / el / 1e9
        if not label:
            out["unit"] = "GB/s"
            out["sample"] = ("%d full pass(es) of the %d-matrix layer at M=%d (quantize + "
                             "integer-route matmul, each matrix's rows split over %d threads, one "
                             "per physical core), %.1f s; the same with 1 thread in value_1core"
                             % (passes, len(wl.matrices), M1, threads, el))
        if M2:
            out["value_m%d%s" % (M2, label)] = ops2 / r["m2"] / 1e12
            if not label:
                out["unit_m%d" % M2] = "TOP/s"
                out["sample_m%d" % M2] = ("%d seeded rows of M=%d (first and last included) "
                                          "through all %d matrices, %.1f s (1 thread: value_m%d_1core)"
                                          % (nrows, M2, len(wl.matrices), r["m2"], M2))
    from quant_packed_weight_amd import synth

    others = {}
    for name in synth.WORKLOADS:
        if name != wl.name:
            others[name] = _oracle_workload(name, seconds / 40, 8 if "1.7b" in name else 32)
    out["workloads_1core"] = others
    out["quantizer_512x1024_us"] = {
        "1core": round(_oracle_quantizer(512, 1024, seconds / 20, 1), 1),
        "%dcores" % cores: round(_oracle_quantizer(512, 1024, seconds / 20, cores), 1),
        "pages_context": "1087 us -> 55.6 us on a 44-core host (another machine)"}
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py: the packed linear layer runs on one GPU per process (it has no "
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
    # activation widths beyond the workload's own are drawn after its own
    gen = synth.generate(a.workload, Ms=set(Ms))
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

    t_eager, rates = {}, {}
    for M in Ms:
        t_eager[M] = time_passes(layer, M, a.steps, a.warmup, copies, stream)
        progress("M=%d: %.1f us per pass" % (M, t_eager[M] * 1e6))
    for M in Ms:
        rates[M] = kernel_rates(layer, M, a.steps, copies, stream)
        progress("M=%d: launches timed" % M)
    if not a.graph:
        t = t_eager
    else:
        graphs = {M: capture_graphs(layer, M, copies) for M in Ms}
        t = {M: time_graphs(graphs[M], a.steps, a.warmup) for M in Ms}

    M1 = Ms[0]
    M2 = Ms[1] if len(Ms) > 1 else None
    ops = {M: sum(2 * M * m.N * m.K for m in wl.matrices) for M in Ms}

    def traffic(prof):
        """HBM bytes (read + written) per launch, averaged over the pass's launches."""
        if not prof or any("read_bytes" not in v for v in prof["per_launch"].values()):
            return None
        pl = prof["per_launch"].values()
        return round(sum(v["read_bytes"] + v["write_bytes"] for v in pl) / len(pl))

    def roof(M):
        per = rates[M]
        n_l = len(per)
        tot_t = sum(dt for _, dt, _ in per.values())
        fused = [k for k, (_, _, f) in per.items() if f]
        kname = kernel_label(M)
        if fused:
            kname += " (quantizer fused into: %s)" % ", ".join(fused)
        prof = profiled(a.workload, M, layer.launches)
        if M <= 8:
            algo = sum(sum(m.nbytes for m in ms) for ms, _, _ in per.values())
            ach = algo / tot_t / 1e9
            r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(ach / HBM_PEAK_GBS, 4),
                 "traffic": traffic(prof),
                 "algo_bytes_per_launch": round(algo / n_l),
                 "kernel": kname, "launches_per_pass": n_l,
                 "avg_launch_us": round(tot_t / n_l * 1e6, 3),
                 "per_launch_us": {k: round(dt * 1e6, 3) for k, (_, dt, _) in per.items()},
                 "per_launch_GBs": {k: round(sum(m.nbytes for m in ms) / dt / 1e9, 1)
                                    for k, (ms, dt, _) in per.items()}}
        else:
            algo = sum(sum(2 * M * m.N * m.K for m in ms) for ms, _, _ in per.values())
            ach = algo / tot_t / 1e12
            r = {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS,
                 "unit": "TOP/s", "frac": round(ach / INT8_PEAK_TOPS, 4),
                 "traffic": traffic(prof),
                 "algo_ops_per_launch": round(algo / n_l),
                 "kernel": kname, "launches_per_pass": n_l,
                 "avg_launch_us": round(tot_t / n_l * 1e6, 3),
                 "per_launch_us": {k: round(dt * 1e6, 3) for k, (_, dt, _) in per.items()},
                 "per_launch_TOPs": {k: round(sum(2 * M * m.N * m.K for m in ms) / dt / 1e12, 1)
                                     for k, (ms, dt, _) in per.items()}}
        r["timing"] = ("HIP events on the launch stream around %d+ back-to-back launches of "
                       "each launch, over >= 1 GiB of rotating weight copies" % a.steps)
        if prof:
            # the same launches' durations in the committed rocprofv3 kernel trace
            pl = prof["per_launch"]
            p_t = sum(v["us"] for v in pl.values()) * 1e-6
            p_ach = algo / p_t / (1e9 if M <= 8 else 1e12)
            r["rocprof"] = {"avg_launch_us": round(p_t / n_l * 1e6, 3),
                            "achieved": round(p_ach, 1),
                            "frac": round(p_ach / r["peak"], 4),
                            "events_over_rocprof_time": round(tot_t / p_t, 4),
                            "per_launch_us": {k: v["us"] for k, v in pl.items()},
                            "source": prof["summary"]}
        else:
            r["rocprof"] = None
        return r

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
        k_t = sum(dt for _, dt, _ in rates[M2].values())
        res["secondary"] = {"metric": "int8 TOP/s at M=%d" % M2,
                            "value": round(ops[M2] / t[M2] / 1e12, 1), "unit": "TOP/s",
                            "frac": round(ops[M2] / t[M2] / 1e12 / INT8_PEAK_TOPS, 4),
                            "matmul_kernels_only_TOPs": round(ops[M2] / k_t / 1e12, 1),
                            "pass_over_matmul_kernels": round(t[M2] / k_t, 4)}
        res["roofline_m%d" % M2] = roof(M2)
    for M in Ms[2:]:
        # the rest of the M sweep: batched decode (weight GB/s) or prefill (int8 TOP/s)
        per = rates[M]
        k_t = sum(dt for _, dt, _ in per.values())
        rec = {"M": M, "kernel": kernel_label(M), "us_per_pass": round(t[M] * 1e6, 2),
               "weight_GBs": round(wbytes / t[M] / 1e9, 1),
               "int8_TOPs": round(ops[M] / t[M] / 1e12, 2),
               "matmul_kernels_us": round(k_t * 1e6, 2)}
        rec["per_launch_us"] = {k: round(dt * 1e6, 3) for k, (_, dt, _) in per.items()}
        if M <= 16:
            rec["per_launch_GBs"] = {k: round(sum(m.nbytes for m in ms) / dt / 1e9, 1)
                                     for k, (ms, dt, _) in per.items()}
            rec["matmul_kernels_frac_of_hbm_peak"] = round(wbytes / k_t / 1e9 / HBM_PEAK_GBS, 4)
            res["batched_decode_m%d" % M] = rec
        else:
            rec["per_launch_TOPs"] = {k: round(sum(2 * M * m.N * m.K for m in ms) / dt / 1e12, 1)
                                      for k, (ms, dt, _) in per.items()}
            rec["matmul_kernels_frac_of_int8_peak"] = round(ops[M] / k_t / 1e12 / INT8_PEAK_TOPS, 4)
            res["prefill_m%d" % M] = rec
    # the standalone activation quantizer at the prefill widths (at M <= 4 with
    # rows of <= 16 blocks it runs fused into the GEMV workgroups instead)
    qrec = {}
    for M in Ms:
        if M > 8:
            q = quantizer_rates(layer, M, a.steps, stream)
            tb = sum(v["algo_bytes"] for v in q.values())
            tt = sum(v["us"] for v in q.values()) * 1e-6
            qrec["M=%d" % M] = {"per_launch": q, "GBs": round(tb / tt / 1e9, 1),
                                "frac": round(tb / tt / 1e9 / HBM_PEAK_GBS, 4)}
    if qrec:
        qrec["kernel"] = "quantize_q8K_kernel"
        qrec["bound"] = "hbm"
        qrec["algo_bytes"] = "M*K*4 (f32 read) + M*(K/256)*292 (q8_K written)"
        qrec["timing"] = ("HIP events around back-to-back launches over >= 1 GiB of rotating "
                          "input copies")
        res["quantizer"] = qrec
    progress("quantizer timed")
    c = res["ceilings"] = measured_ceilings(
        wl, {launch_name(ms): sum(m.nbytes for m in ms) for ms in layer.launches})
    progress("ceilings measured")
    c["read_frac_of_peak"] = round(c["read_GBs"] / HBM_PEAK_GBS, 4)
    c["copy_frac_of_peak"] = round(c["copy_GBs"] / HBM_PEAK_GBS, 4)
    c["mfma_i8_frac_of_peak"] = round(c["mfma_i8_TOPs"] / INT8_PEAK_TOPS, 4)
    if c.get("int8_gemm_TOPs"):
        c["int8_gemm_frac_of_peak"] = round(c["int8_gemm_TOPs"] / INT8_PEAK_TOPS, 4)
    # the kernels against the measured ceilings as well as the datasheet peaks
    for key in ["roofline"] + (["roofline_m%d" % M2] if M2 else []):
        r = res[key]
        if r["bound"] == "hbm":
            r["frac_of_measured_read"] = round(r["achieved"] / c["read_GBs"], 4)
            r["per_launch_frac_of_measured_read"] = {
                k: round(v / c["read_GBs"], 4) for k, v in r["per_launch_GBs"].items()}
            r["per_launch_frac_of_peak"] = {
                k: round(v / HBM_PEAK_GBS, 4) for k, v in r["per_launch_GBs"].items()}
            rs = c.get("read_same_bytes", {})
            if all(k in rs for k in r["per_launch_us"]):
                # against a plain read of each launch's bytes (fixed launch costs in both)
                r["per_launch_frac_of_same_size_read"] = {
                    k: round(rs[k]["us"] / v, 4) for k, v in r["per_launch_us"].items()}
                r["frac_of_same_size_read"] = round(
                    sum(rs[k]["us"] for k in r["per_launch_us"]) / sum(r["per_launch_us"].values()), 4)
        else:
            r["frac_of_measured_mfma"] = round(r["achieved"] / c["mfma_i8_TOPs"], 4)
            if c.get("int8_gemm_TOPs"):
                r["vs_int8_gemm_library"] = round(r["achieved"] / c["int8_gemm_TOPs"], 4)
    if not a.no_other_workloads:
        res["other_workloads"] = other_workloads(a.workload, a.steps, a.warmup)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, gen, M1, M2, a.cpu_seconds)
        progress("oracle timed")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
