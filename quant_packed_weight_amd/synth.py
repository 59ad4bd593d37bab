"""Seeded synthetic inputs shaped like the PocketLLM pages' Qwen3 workloads.

This module only draws random bytes and floats and places them in the block
fields; it holds none of the method's arithmetic (no decode, no quantization, no
dot product), so both the HIP path and the CPU oracle can consume its output.

Distributions (the pages measure Qwen3-0.6B/1.7B checkpoints, which are not
available here; these stand in for them):
  q4_K: d and dmin = f16(|N(0,1)| * 2e-3); the 12 scale/min bytes and the 128
        quant bytes are uniform random bytes, which makes every 6-bit scale and
        min uniform on 0..63 and every 4-bit quant uniform on 0..15.
  q6_K: low-nibble and high-bit bytes uniform random (quants uniform on 0..63);
        sub-scales uniform on -64..63; d = f16(|N(0,1)| * 1e-3).
  q2_K, q5_K: as q4_K (uniform scale/min and quant bytes, d and dmin =
        f16(|N(0,1)| * 2e-3)); q2_K's 4-bit scales and mins and 2-bit quants, q5_K's
        6-bit scales and mins and 5-bit quants are then uniform.
  q3_K: uniform mask, quant and scale bytes (6-bit scales uniform on 0..63,
        i.e. -32..31 after the offset; quants uniform on -4..3);
        d = f16(|N(0,1)| * 2e-3).
  activations: f32 N(0,1); optionally 4 distinct outlier columns (the same in
        every row) multiplied by 20.
Draw order per workload: every matrix's weight bytes in list order, then the
activations for each M in order, one tensor per distinct input of the layer
(attention input, attention output, MLP input, MLP activation, final hidden
state) in order of first use.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FMT_Q2K = 10  # GGUF type ids
FMT_Q3K = 11
FMT_Q4K = 12
FMT_Q5K = 13
FMT_Q6K = 14
BLOCK_BYTES = {FMT_Q2K: 84, FMT_Q3K: 110, FMT_Q4K: 144, FMT_Q5K: 176, FMT_Q6K: 210}
FMT_NAME = {FMT_Q2K: "q2_K", FMT_Q3K: "q3_K", FMT_Q4K: "q4_K", FMT_Q5K: "q5_K",
            FMT_Q6K: "q6_K"}
# byte offsets of the f16 factors d and dmin in each block
_D_OFFS = {FMT_Q2K: (80, 82), FMT_Q3K: (108,), FMT_Q4K: (0, 2), FMT_Q5K: (0, 2)}
Q8K_BYTES = 292
QK = 256


@dataclass(frozen=True)
class Matrix:
    name: str
    N: int  # output rows
    K: int  # inputs
    fmt: int
    inp: str = "x"  # name of the activation tensor this matrix reads

    @property
    def nbytes(self) -> int:
        return self.N * (self.K // QK) * BLOCK_BYTES[self.fmt]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    matrices: tuple
    Ms: tuple
    outliers: bool = True
    doc: str = ""

    def inputs(self):
        """Distinct activation tensors in order of first use: [(name, K)]."""
        out = []
        for m in self.matrices:
            if (m.inp, m.K) not in out:
                out.append((m.inp, m.K))
        return out


def _qwen3(hidden, heads_dim, kv_dim, inter, fmts, head=None):
    q4, q6 = FMT_Q4K, FMT_Q6K
    # q/k/v read the attention input, o the attention output, gate/up the MLP
    # input, down the gated MLP activation, the head the final hidden state
    mats = [
        Matrix("q_proj", heads_dim, hidden, fmts.get("q", q4), "attn_in"),
        Matrix("k_proj", kv_dim, hidden, fmts.get("k", q4), "attn_in"),
        Matrix("v_proj", kv_dim, hidden, fmts.get("v", q4), "attn_in"),
        Matrix("o_proj", hidden, heads_dim, fmts.get("o", q4), "attn_out"),
        Matrix("gate_proj", inter, hidden, fmts.get("gate", q4), "mlp_in"),
        Matrix("up_proj", inter, hidden, fmts.get("up", q4), "mlp_in"),
        Matrix("down_proj", hidden, inter, fmts.get("down", q4), "mlp_act"),
    ]
    if head:
        mats.append(Matrix("output", head, hidden, fmts.get("head", q4), "final"))
    return tuple(mats)


_MIX = {"v": FMT_Q6K, "down": FMT_Q6K, "head": FMT_Q6K}  # q4_K_M mix: v/down/head in q6_K

WORKLOADS = {
    "q4K-1024x1024-m8": Workload(
        "q4K-1024x1024-m8", 0, (Matrix("w", 1024, 1024, FMT_Q4K),), (8,), outliers=False,
        doc="one q4_K matrix, N=K=1024, M=8"),
    "qwen3-0.6b-decode": Workload(
        "qwen3-0.6b-decode", 1, _qwen3(1024, 2048, 1024, 3072, _MIX), (1,),
        doc="Qwen3-0.6B layer GEMV set, q4_K_M mix, M=1"),
    "qwen3-0.6b-prefill512": Workload(
        "qwen3-0.6b-prefill512", 2, _qwen3(1024, 2048, 1024, 3072, _MIX), (512,),
        doc="Qwen3-0.6B layer GEMM set, q4_K_M mix, M=512"),
    "qwen3-1.7b-layer-head": Workload(
        "qwen3-1.7b-layer-head", 3, _qwen3(2048, 2048, 1024, 6144, _MIX, head=151936), (1, 512),
        doc="Qwen3-1.7B layer plus q6_K LM head, q4_K_M mix, M=1 and 512"),
    "qwen3-8b-q4K": Workload(
        "qwen3-8b-q4K", 4, _qwen3(4096, 4096, 1024, 12288, {}), (1, 8, 512, 2048),
        doc="Qwen3-8B-shaped layer, all q4_K, M in 1, 8, 512, 2048"),
}


def make_weights(rng: np.random.Generator, fmt: int, N: int, K: int,
                 d_scale: float | None = None) -> np.ndarray:
    """Random packed weights: uint8 [N, (K/256) * block_bytes]."""
    assert K % QK == 0 and N >= 0
    nblk = N * (K // QK)
    bb = BLOCK_BYTES[fmt]
    raw = rng.integers(0, 256, size=(nblk, bb), dtype=np.uint8)
    if fmt in _D_OFFS:
        s = 2e-3 if d_scale is None else d_scale
        for o in _D_OFFS[fmt]:
            f = (np.abs(rng.standard_normal(nblk)) * s).astype(np.float16)
            raw[:, o:o + 2] = f.view(np.uint8).reshape(nblk, 2)
    elif fmt == FMT_Q6K:
        s = 1e-3 if d_scale is None else d_scale
        sc = rng.integers(-64, 64, size=(nblk, 16)).astype(np.int8)
        raw[:, 192:208] = sc.view(np.uint8)
        d = (np.abs(rng.standard_normal(nblk)) * s).astype(np.float16)
        raw[:, 208:210] = d.view(np.uint8).reshape(nblk, 2)
    else:
        raise ValueError("unknown format %r" % fmt)
    return raw.reshape(N, (K // QK) * bb)


def make_activations(rng: np.random.Generator, M: int, K: int, outliers: bool) -> np.ndarray:
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        cols = rng.choice(K, size=4, replace=False)
        x[:, cols] *= np.float32(20.0)
    return x


@dataclass
class Generated:
    workload: Workload
    weights: dict = field(default_factory=dict)      # matrix name -> uint8 [N, bytes]
    activations: dict = field(default_factory=dict)  # (M, input name) -> f32 [M, K]


def generate(name: str, Ms=None, with_weights: bool = True) -> Generated:
    """Draw a named workload.  ``Ms`` restricts which activation sets are kept,
    without changing the draw order (the others are drawn and dropped); widths
    in ``Ms`` that the workload does not list are drawn after its own."""
    wl = WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    g = Generated(wl)
    for mat in wl.matrices:
        w = make_weights(rng, mat.fmt, mat.N, mat.K)
        if with_weights:
            g.weights[mat.name] = w
        else:
            del w
    for M in wl.Ms:
        for inp, K in wl.inputs():
            x = make_activations(rng, M, K, wl.outliers)
            if Ms is None or M in Ms:
                g.activations[(M, inp)] = x
    # activation widths outside the workload's own, drawn after all of those
    # (so they change none of them), in increasing M
    for M in sorted(set(Ms or ()) - set(wl.Ms)):
        for inp, K in wl.inputs():
            g.activations[(M, inp)] = make_activations(rng, M, K, wl.outliers)
    return g
