"""ctypes front end of ``gemmq_oracle.c`` (test infrastructure only).

The C file is the oracle; this module only builds it with gcc, loads it and moves
numpy arrays in and out.  No arithmetic of the method lives here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemmq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FMT_Q2K = 10
FMT_Q3K = 11
FMT_Q4K = 12
FMT_Q5K = 13
FMT_Q6K = 14
BLOCK_BYTES = {FMT_Q2K: 84, FMT_Q3K: 110, FMT_Q4K: 144, FMT_Q5K: 176, FMT_Q6K: 210}
Q8K_BYTES = 292

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction) into liboracle.so."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-fPIC", "-shared",
           "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
            lib.oracle_f16_to_f64.restype = ctypes.c_double
            lib.oracle_decode_q4K.argtypes = [P, I64, P]
            lib.oracle_decode_q4K.restype = None
            lib.oracle_decode_q6K.argtypes = [P, I64, P]
            lib.oracle_decode_q6K.restype = None
            lib.oracle_decode.argtypes = [ctypes.c_int, P, I64, P]
            lib.oracle_decode.restype = ctypes.c_int
            lib.oracle_quantize_q8K.argtypes = [P, I64, I64, P]
            lib.oracle_quantize_q8K.restype = ctypes.c_int
            lib.oracle_gemm_int.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P, I64, P]
            lib.oracle_gemm_int.restype = ctypes.c_int
            lib.oracle_gemm_dequant.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P, I64, P, P]
            lib.oracle_gemm_dequant.restype = ctypes.c_int
            lib.oracle_repack.argtypes = [ctypes.c_int, P, I64, I64, P]
            lib.oracle_repack.restype = ctypes.c_int
            lib.oracle_silu_mul.argtypes = [P, P, I64, P]
            lib.oracle_silu_mul.restype = None
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def f16_to_f64(h: int) -> float:
    return load().oracle_f16_to_f64(int(h) & 0xFFFF)


def decode(fmt: int, W: np.ndarray, N: int, K: int) -> np.ndarray:
    """Packed weights (N rows of K/256 blocks, raw bytes) -> f32 [N, K]."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    nblk = N * (K // 256)
    assert W.size == nblk * BLOCK_BYTES[fmt]
    out = np.empty((N, K), dtype=np.float32)
    if fmt == FMT_Q4K:
        load().oracle_decode_q4K(_ptr(W), nblk, _ptr(out))
    elif fmt == FMT_Q6K:
        load().oracle_decode_q6K(_ptr(W), nblk, _ptr(out))
    elif load().oracle_decode(fmt, _ptr(W), nblk, _ptr(out)) != 0:
        raise ValueError("oracle_decode: unknown format %d" % fmt)
    return out


def quantize_q8K(X: np.ndarray) -> np.ndarray:
    """f32 [M, K] -> q8_K bytes [M, K/256 * 292]."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    M, K = X.shape
    out = np.zeros((M, (K // 256) * Q8K_BYTES), dtype=np.uint8)
    rc = load().oracle_quantize_q8K(_ptr(X), M, K, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_quantize_q8K: K must be a multiple of 256")
    return out


def _rows_arg(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < M))
    return r, r.size


def gemm_int(fmt, W, Xq, M, N, K, rows=None) -> np.ndarray:
    """Integer-decomposition route: float64 [len(rows) or M, N]."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    r, nr = _rows_arg(rows, M)
    Y = np.empty((nr, N), dtype=np.float64)
    rc = load().oracle_gemm_int(fmt, _ptr(W), _ptr(Xq), M, N, K, _ptr(r), nr, _ptr(Y))
    if rc != 0:
        raise ValueError("oracle_gemm_int: bad arguments")
    return Y


def gemm_dequant(fmt, W, Xq, M, N, K, rows=None):
    """Decode-then-dot route and error scale: (Y, S), float64 [rows, N] each."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    r, nr = _rows_arg(rows, M)
    Y = np.empty((nr, N), dtype=np.float64)
    S = np.empty((nr, N), dtype=np.float64)
    rc = load().oracle_gemm_dequant(fmt, _ptr(W), _ptr(Xq), M, N, K, _ptr(r), nr, _ptr(Y),
                                    _ptr(S))
    if rc != 0:
        raise ValueError("oracle_gemm_dequant: bad arguments")
    return Y, S


def silu_mul(g, u) -> np.ndarray:
    """silu(g) * u element by element, float64 (same shape as g)."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    assert g.shape == u.shape
    y = np.empty_like(g)
    load().oracle_silu_mul(_ptr(g), _ptr(u), g.size, _ptr(y))
    return y


def repack(fmt: int, W: np.ndarray, N: int, K: int) -> np.ndarray:
    """q3_K / q6_K matrix -> its load-time repacked bytes (same size, uint8 [N, row bytes])."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    assert W.size == N * (K // 256) * BLOCK_BYTES[fmt]
    out = np.empty_like(W).reshape(N, -1)
    if load().oracle_repack(fmt, _ptr(W), N, K, _ptr(out)) != 0:
        raise ValueError("oracle_repack: format %d has no repacked layout" % fmt)
    return out
