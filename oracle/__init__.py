"""CPU oracle for the packed-weight linear layer.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product package never imports it.
"""
from .oracle import (  # noqa: F401
    FMT_Q2K,
    FMT_Q3K,
    FMT_Q4K,
    FMT_Q5K,
    FMT_Q6K,
    build,
    decode,
    f16_to_f64,
    gemm_dequant,
    gemm_int,
    load,
    quantize_q8K,
    repack,
    silu_mul,
)
