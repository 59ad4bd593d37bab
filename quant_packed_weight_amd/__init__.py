"""quant_packed_weight_amd -- libgemmq, the packed-weight linear layer on MI355X.

The HIP library (libgemmq.so, C ABI in include/gemmq.h) computes y = W x on ggml
q4_K / q6_K packed weights with q8_K-quantized activations; this package is its
thin ctypes binding plus the seeded synthetic input generator (``synth``).
The library is loaded on first use; nothing here computes on the CPU.
"""
from ._lib import (  # noqa: F401
    ABI_VERSION,
    BLOCK_BYTES,
    EXPORTS,
    FMT_Q2K,
    FMT_Q3K,
    FMT_Q3K_R,
    FMT_Q4K,
    FMT_Q5K,
    FMT_Q6K,
    FMT_Q6K_R,
    GEMM_MAX_M,
    LIB_PATH,
    MAX_GROUP,
    PATH_AUTO,
    PATH_GEMM,
    PATH_GEMV,
    PATH_SKINNY,
    PROBE_CHAINS,
    PROBE_MAX_ITERS,
    PROBE_READ_WORDS,
    Q8K_BYTES,
    QK,
    GemmqError,
    block_bytes,
    decode,
    decode_ptr,
    gemm,
    gemm_group,
    gemm_group_ptr,
    gemm_ptr,
    lib,
    linear,
    linear_group,
    linear_group_ptr,
    linear_silu_mul,
    probe_mfma_i8,
    probe_mfma_valu,
    probe_read,
    q8K_bytes,
    quantize_q8K,
    repack,
    quantize_q8K_ptr,
    status_str,
    weight_bytes,
)

__version__ = "0.1.0"
