"""ctypes binding of libgemmq (include/gemmq.h).

Argument marshalling only: every step of the computation runs in the HIP kernels
of libgemmq.so.  Torch supplies device memory and the current stream.  There is
no fallback: if the library is missing or the device is not a gfx950, calls
raise GemmqError.
"""
from __future__ import annotations

import ctypes
import os
import threading

FMT_Q2K = 10
FMT_Q3K = 11
FMT_Q4K = 12
FMT_Q5K = 13
FMT_Q6K = 14
FMT_Q3K_R = 256 + FMT_Q3K  # repacked layouts (gemmq_repack)
FMT_Q6K_R = 256 + FMT_Q6K
BLOCK_BYTES = {FMT_Q2K: 84, FMT_Q3K: 110, FMT_Q4K: 144, FMT_Q5K: 176, FMT_Q6K: 210,
               FMT_Q3K_R: 110, FMT_Q6K_R: 210}
Q8K_BYTES = 292
QK = 256
PATH_AUTO, PATH_GEMV, PATH_GEMM, PATH_SKINNY = 0, 1, 2, 3
MAX_GROUP = 4  # matrices per gemmq_gemm_group / gemmq_linear_group call
ABI_VERSION = 10
PROBE_CHAINS = 4  # GEMMQ_PROBE_CHAINS
PROBE_MAX_ITERS = 1000000  # GEMMQ_PROBE_MAX_ITERS
GEMM_MAX_M = 4194240  # GEMMQ_GEMM_MAX_M
PROBE_READ_WORDS = 2048  # GEMMQ_PROBE_READ_WORDS

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemmq.so")

# every entry point include/gemmq.h declares: name -> (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
EXPORTS = {
    "gemmq_abi_version": (_I, []),
    "gemmq_status_str": (ctypes.c_char_p, [_I]),
    "gemmq_block_bytes": (ctypes.c_size_t, [_I]),
    "gemmq_weight_bytes": (ctypes.c_size_t, [_I, _I64, _I64]),
    "gemmq_q8K_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "gemmq_quantize_q8K": (_I, [_P, _P, _I64, _I64, _P]),
    "gemmq_gemm": (_I, [_I, _P, _P, _P, _I64, _I64, _I64, _P]),
    "gemmq_gemm_ex": (_I, [_I, _P, _P, _P, _I64, _I64, _I64, _I, _P]),
    "gemmq_gemm_group": (_I, [_I, _I, ctypes.POINTER(_P), ctypes.POINTER(_P),
                              ctypes.POINTER(_I64), _P, _I64, _I64, _I, _P]),
    "gemmq_linear_group": (_I, [_I, _I, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                ctypes.POINTER(_I64), _P, _P, _I64, _I64, _I, _P]),
    "gemmq_linear": (_I, [_I, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "gemmq_linear_silu_mul": (_I, [_I, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P]),
    "gemmq_decode": (_I, [_I, _P, _P, _I64, _I64, _P]),
    "gemmq_repack": (_I, [_I, _P, _P, _I64, _I64, _P]),
    "gemmq_probe_mfma_i8": (_I, [_I64, _I64, _P, _P, _P]),
    "gemmq_probe_mfma_valu": (_I, [_I64, _I64, _I, _P, _P, _P]),
    "gemmq_probe_read": (_I, [_P, _I64, _P, _P]),
}


class GemmqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = status_str(status) if _lib is not None else str(status)
        super().__init__("%s: %s" % (where, name))


_lib = None
_lock = threading.Lock()


def lib():
    """Load libgemmq.so once (raises GemmqError(-100) when it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise GemmqError(-100, "libgemmq.so is not built (%s); run "
                                       "python -m quant_packed_weight_amd.build" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in EXPORTS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            if L.gemmq_abi_version() != ABI_VERSION:
                raise GemmqError(-101, "libgemmq ABI %d, binding expects %d"
                                 % (L.gemmq_abi_version(), ABI_VERSION))
            _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().gemmq_status_str(int(status)).decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise GemmqError(rc, where)


def block_bytes(fmt: int) -> int:
    return lib().gemmq_block_bytes(fmt)


def weight_bytes(fmt: int, N: int, K: int) -> int:
    return lib().gemmq_weight_bytes(fmt, N, K)


def q8K_bytes(M: int, K: int) -> int:
    return lib().gemmq_q8K_bytes(M, K)


# ------------------------------------------------------------ raw-pointer calls
def quantize_q8K_ptr(X: int, Xq: int, M: int, K: int, stream: int = 0) -> int:
    return lib().gemmq_quantize_q8K(X, Xq, M, K, stream or None)


def gemm_ptr(fmt: int, W: int, Xq: int, Y: int, M: int, N: int, K: int, path: int = PATH_AUTO,
             stream: int = 0) -> int:
    return lib().gemmq_gemm_ex(fmt, W, Xq, Y, M, N, K, path, stream or None)


def gemm_group_ptr(fmt: int, Ws, Ys, Ns, Xq: int, M: int, K: int, path: int = PATH_AUTO,
                   stream: int = 0) -> int:
    """Ws, Ys, Ns: sequences of equal length (the matrices sharing Xq)."""
    n = len(Ws)
    if len(Ys) != n or len(Ns) != n:
        raise ValueError("Ws, Ys and Ns must have the same length")
    wa = (_P * max(n, 1))(*Ws)
    ya = (_P * max(n, 1))(*Ys)
    na = (_I64 * max(n, 1))(*Ns)
    return lib().gemmq_gemm_group(fmt, n, wa, ya, na, Xq, M, K, path, stream or None)


def linear_group_ptr(fmt: int, Ws, Ys, Ns, X: int, Xq: int, M: int, K: int,
                     path: int = PATH_AUTO, stream: int = 0) -> int:
    """Quantize X into Xq and apply the matrices Ws (gemmq_linear_group)."""
    n = len(Ws)
    if len(Ys) != n or len(Ns) != n:
        raise ValueError("Ws, Ys and Ns must have the same length")
    wa = (_P * max(n, 1))(*Ws)
    ya = (_P * max(n, 1))(*Ys)
    na = (_I64 * max(n, 1))(*Ns)
    return lib().gemmq_linear_group(fmt, n, wa, ya, na, X, Xq, M, K, path, stream or None)


def decode_ptr(fmt: int, W: int, Wf: int, N: int, K: int, stream: int = 0) -> int:
    return lib().gemmq_decode(fmt, W, Wf, N, K, stream or None)


# ------------------------------------------------------------ torch-tensor calls
def _torch():
    import torch

    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t, name, dtype):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def quantize_q8K(x, out=None, stream=None):
    """f32 [M, K] device tensor -> uint8 [M, K/256*292] q8_K blocks."""
    torch = _torch()
    M, K = x.shape
    if out is None:
        out = torch.empty((M, (K // QK) * Q8K_BYTES), dtype=torch.uint8, device=x.device)
    elif out.numel() < q8K_bytes(M, K):
        raise ValueError("out too small")
    _check(lib().gemmq_quantize_q8K(_dev(x, "x", torch.float32), _dev(out, "out", torch.uint8),
                                    M, K, _stream(stream)), "gemmq_quantize_q8K")
    return out


def gemm(fmt, w, xq, M, N, K, out=None, path=PATH_AUTO, stream=None):
    """Packed weights (uint8) x q8_K activations (uint8) -> f32 [M, N]."""
    torch = _torch()
    if w.numel() < weight_bytes(fmt, N, K) or xq.numel() < q8K_bytes(M, K):
        raise ValueError("buffer smaller than the stated shape")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    elif out.numel() < M * N:
        raise ValueError("out too small")
    _check(lib().gemmq_gemm_ex(fmt, _dev(w, "w", torch.uint8), _dev(xq, "xq", torch.uint8),
                               _dev(out, "out", torch.float32), M, N, K, path, _stream(stream)),
           "gemmq_gemm")
    return out


def gemm_group(fmt, ws, xq, M, Ns, K, outs=None, path=PATH_AUTO, stream=None):
    """Several packed weight matrices sharing the activations xq, one launch:
    returns [f32 [M, N_g]]."""
    torch = _torch()
    if len(ws) != len(Ns):
        raise ValueError("ws and Ns must have the same length")
    if xq.numel() < q8K_bytes(M, K):
        raise ValueError("xq smaller than the stated shape")
    for w, N in zip(ws, Ns):
        if w.numel() < weight_bytes(fmt, N, K):
            raise ValueError("buffer smaller than the stated shape")
    if outs is None:
        outs = [torch.empty((M, N), dtype=torch.float32, device=xq.device) for N in Ns]
    for o, N in zip(outs, Ns):
        if o.numel() < M * N:
            raise ValueError("out too small")
    _check(gemm_group_ptr(fmt, [_dev(w, "w", torch.uint8) for w in ws],
                          [_dev(o, "out", torch.float32) for o in outs], list(Ns),
                          _dev(xq, "xq", torch.uint8), M, K, path, _stream(stream)),
           "gemmq_gemm_group")
    return outs


def decode(fmt, w, N, K, out=None, stream=None):
    """Packed weights -> f32 [N, K] (diagnostic)."""
    torch = _torch()
    if w.numel() < weight_bytes(fmt, N, K):
        raise ValueError("w smaller than the stated shape")
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=w.device)
    elif out.numel() < N * K:
        raise ValueError("out too small")
    _check(lib().gemmq_decode(fmt, _dev(w, "w", torch.uint8), _dev(out, "out", torch.float32),
                              N, K, _stream(stream)), "gemmq_decode")
    return out


def linear_group(fmt, ws, x, Ns, xq=None, outs=None, path=PATH_AUTO, stream=None):
    """f32 activations x [M, K] through several packed matrices (gemmq_linear_group):
    returns ([f32 [M, N_g]], xq) with xq the q8_K blocks of x."""
    torch = _torch()
    M, K = x.shape
    if len(ws) != len(Ns):
        raise ValueError("ws and Ns must have the same length")
    for w, N in zip(ws, Ns):
        if w.numel() < weight_bytes(fmt, N, K):
            raise ValueError("buffer smaller than the stated shape")
    if xq is None:
        xq = torch.empty((M, (K // QK) * Q8K_BYTES), dtype=torch.uint8, device=x.device)
    elif xq.numel() < q8K_bytes(M, K):
        raise ValueError("xq too small")
    if outs is None:
        outs = [torch.empty((M, N), dtype=torch.float32, device=x.device) for N in Ns]
    for o, N in zip(outs, Ns):
        if o.numel() < M * N:
            raise ValueError("out too small")
    _check(linear_group_ptr(fmt, [_dev(w, "w", torch.uint8) for w in ws],
                            [_dev(o, "out", torch.float32) for o in outs], list(Ns),
                            _dev(x, "x", torch.float32), _dev(xq, "xq", torch.uint8), M, K, path,
                            _stream(stream)), "gemmq_linear_group")
    return outs, xq


def linear(fmt, w, x, N, path=PATH_AUTO, stream=None):
    """y = W x for f32 activations x [M, K] (quantized to q8_K on the device)."""
    outs, _ = linear_group(fmt, [w], x, [N], path=path, stream=stream)
    return outs[0]


def linear_silu_mul(fmt, wg, wu, x, N, xq=None, out=None, path=PATH_AUTO, stream=None):
    """silu(Wg x) * (Wu x) for f32 activations x [M, K] (gemmq_linear_silu_mul):
    returns (f32 [M, N], xq) with xq the q8_K blocks of x."""
    torch = _torch()
    M, K = x.shape
    for w in (wg, wu):
        if w.numel() < weight_bytes(fmt, N, K):
            raise ValueError("buffer smaller than the stated shape")
    if xq is None:
        xq = torch.empty((M, (K // QK) * Q8K_BYTES), dtype=torch.uint8, device=x.device)
    elif xq.numel() < q8K_bytes(M, K):
        raise ValueError("xq too small")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    elif out.numel() < M * N:
        raise ValueError("out too small")
    _check(lib().gemmq_linear_silu_mul(fmt, _dev(wg, "wg", torch.uint8), _dev(wu, "wu", torch.uint8),
                                       _dev(x, "x", torch.float32), _dev(xq, "xq", torch.uint8),
                                       _dev(out, "out", torch.float32), M, N, K, path,
                                       _stream(stream)), "gemmq_linear_silu_mul")
    return out, xq


def repack(fmt, w, N, K, out=None, stream=None):
    """q3_K / q6_K weights (uint8 device tensor) -> their repacked layout
    (gemmq_repack); use the result with FMT_Q3K_R / FMT_Q6K_R."""
    torch = _torch()
    nbytes = weight_bytes(fmt, N, K)
    if w.numel() < nbytes:
        raise ValueError("buffer smaller than the stated shape")
    if out is None:
        out = torch.empty((N, nbytes // max(N, 1)), dtype=torch.uint8, device=w.device)
    elif out.numel() < nbytes:
        raise ValueError("out too small")
    _check(lib().gemmq_repack(fmt, _dev(w, "w", torch.uint8), _dev(out, "out", torch.uint8), N, K,
                              _stream(stream)), "gemmq_repack")
    return out


def probe_mfma_i8(iters, blocks, stream=None):
    """Enqueue the int8 MFMA ceiling loop (gemmq_probe_mfma_i8); returns the
    (out, clocks) device tensors and the int8 operation count of the launch."""
    torch = _torch()
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    _check(lib().gemmq_probe_mfma_i8(iters, blocks, out.data_ptr(), clocks.data_ptr(),
                                     _stream(stream)), "gemmq_probe_mfma_i8")
    return out, clocks, 2 * 32768 * PROBE_CHAINS * 4 * blocks * iters


def probe_mfma_valu(iters, blocks, valu, stream=None):
    """Enqueue the int8 MFMA loop with `valu` f32 FMAs after every MFMA
    (gemmq_probe_mfma_valu); returns (out, clocks) and the int8 operation
    count of the launch."""
    torch = _torch()
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    _check(lib().gemmq_probe_mfma_valu(iters, blocks, valu, out.data_ptr(), clocks.data_ptr(),
                                       _stream(stream)), "gemmq_probe_mfma_valu")
    return out, clocks, 2 * 32768 * PROBE_CHAINS * 4 * blocks * iters


def probe_read(src, stream=None):
    """Enqueue the read-only stream over the device tensor `src`
    (gemmq_probe_read); returns the per-wave fold tensor."""
    torch = _torch()
    out = torch.empty(PROBE_READ_WORDS, dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size()
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _check(lib().gemmq_probe_read(src.data_ptr(), nbytes - nbytes % 16, out.data_ptr(),
                                  _stream(stream)), "gemmq_probe_read")
    return out
