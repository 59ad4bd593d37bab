"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments with a named status before it
touches the device.  Every call below fails validation, so none reaches HIP.
"""
import ctypes
import os
import re
import subprocess

import pytest

import quant_packed_weight_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemmq.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gemmq_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gq.LIB_PATH):
        pytest.fail("libgemmq.so not built: run python -m quant_packed_weight_amd.build")
    return gq.lib()


def test_every_declared_symbol_exported(L):
    names = _declared()
    assert len(names) == 17
    assert set(names) == set(gq.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", gq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(gemmq_\w+)", out))
    assert set(names) <= exported
    for n in names:
        assert getattr(L, n) is not None


def test_version_and_status_names(L):
    assert L.gemmq_abi_version() == gq.ABI_VERSION == 10
    for code, word in [(0, "GEMMQ_OK"), (-1, "INVALID_ARG"), (-2, "UNSUPPORTED_FORMAT"),
                       (-3, "SHAPE"), (-4, "ALIGNMENT"), (-5, "DEVICE"), (-6, "LAUNCH"),
                       (-77, "UNKNOWN")]:
        assert word in gq.status_str(code)


def test_size_helpers(L):
    assert [gq.block_bytes(f) for f in range(9, 16)] == [0, 84, 110, 144, 176, 210, 0]
    assert [gq.block_bytes(256 + f) for f in range(9, 16)] == [0, 0, 110, 0, 0, 210, 0]
    assert gq.weight_bytes(12, 4096, 4096) == 4096 * 16 * 144
    assert gq.weight_bytes(14, 151936, 2048) == 255252480
    assert gq.weight_bytes(12, 10, 300) == 0 and gq.weight_bytes(12, -1, 256) == 0
    assert gq.weight_bytes(99, 10, 256) == 0
    assert gq.q8K_bytes(512, 1024) == 598016
    assert gq.q8K_bytes(1, 12288) == 14016
    assert gq.q8K_bytes(1, 100) == 0 and gq.q8K_bytes(-1, 256) == 0


FAKE16 = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,status", [
    ((15, FAKE16, FAKE16, FAKE16, 1, 1, 256, 0), -2),      # unknown format
    ((9, FAKE16, FAKE16, FAKE16, 1, 1, 256, 0), -2),       # unknown format
    ((13, FAKE16 + 4, FAKE16, FAKE16, 1, 1, 256, 0), -4),  # q5_K weights need 16 bytes
    ((10, FAKE16 + 2, FAKE16, FAKE16, 1, 1, 256, 0), -4),  # q2_K weights need 4 bytes
    ((11, FAKE16 + 2, FAKE16, FAKE16, 1, 1, 256, 0), -4),  # q3_K weights need 4 bytes
    ((12, FAKE16, FAKE16, FAKE16, 1, 1, 300, 0), -3),      # K % 256 != 0
    ((12, FAKE16, FAKE16, FAKE16, 1, 1, 0, 0), -3),        # K = 0
    ((12, FAKE16, FAKE16, FAKE16, 1, -1, 256, 0), -1),     # N < 0
    ((12, FAKE16, FAKE16, FAKE16, -1, 1, 256, 0), -1),     # M < 0
    ((12, None, FAKE16, FAKE16, 1, 1, 256, 0), -1),        # null W
    ((12, FAKE16, None, FAKE16, 1, 1, 256, 0), -1),        # null Xq
    ((12, FAKE16, FAKE16, None, 1, 1, 256, 0), -1),        # null Y
    ((12, FAKE16 + 4, FAKE16, FAKE16, 1, 1, 256, 0), -4),  # q4_K weights need 16 B
    ((14, FAKE16 + 2, FAKE16, FAKE16, 1, 1, 256, 0), -4),  # q6_K weights need 4 B
    ((12, FAKE16, FAKE16 + 2, FAKE16, 1, 1, 256, 0), -4),  # Xq needs 4 B
    ((12, FAKE16, FAKE16, FAKE16 + 1, 1, 1, 256, 0), -4),  # Y needs 4 B
    ((12, FAKE16, FAKE16, FAKE16, 1, 1, 256, 7), -1),      # unknown path
    ((12, FAKE16, FAKE16, FAKE16, 9, 1, 256, 1), -3),      # GEMV path with M > 8
    ((12, FAKE16, FAKE16, FAKE16, 65, 1, 256, 3), -3),     # small-M MFMA path with M > 64
    ((14, FAKE16, FAKE16, FAKE16, 17, 1, 256, 3), -3),     # small-M MFMA path: q6_K M <= 16
    ((270, FAKE16, FAKE16, FAKE16, 17, 1, 256, 3), -3),
    ((13, FAKE16, FAKE16, FAKE16, 4, 1, 256, 3), -2),      # small-M MFMA path: q4_K, q6_K only
    ((10, FAKE16, FAKE16, FAKE16, 4, 1, 256, 3), -2),
    ((11, FAKE16, FAKE16, FAKE16, 4, 1, 256, 3), -2),
    ((12, FAKE16, FAKE16, FAKE16, 0, 5, 256, 0), 0),       # M = 0: empty, nothing touched
    ((12, FAKE16, FAKE16, FAKE16, 5, 0, 256, 0), 0),       # N = 0: empty
    ((12, FAKE16, FAKE16, FAKE16, gq.GEMM_MAX_M + 1, 1, 256, 2), -3),  # GEMM grid limit
    ((12, FAKE16, FAKE16, FAKE16, gq.GEMM_MAX_M + 1, 1, 256, 0), -3),  # the same, chosen
    ((14, FAKE16, FAKE16, FAKE16, gq.GEMM_MAX_M + 1, 1, 256, 0), -3),
])
def test_gemm_validation(L, args, status):
    fmt, W, Xq, Y, M, N, K, path = args
    assert L.gemmq_gemm_ex(fmt, W, Xq, Y, M, N, K, path, None) == status
    if path == 0:
        assert L.gemmq_gemm(fmt, W, Xq, Y, M, N, K, None) == status


@pytest.mark.parametrize("count,Ws,Ys,Ns,M,path,status", [
    (0, [FAKE16], [FAKE16], [1], 1, 0, -1),                           # count < 1
    (5, [FAKE16] * 5, [FAKE16] * 5, [1] * 5, 1, 0, -1),               # count > 4
    (2, [FAKE16, None], [FAKE16, FAKE16], [1, 1], 1, 0, -1),          # null W in entry 1
    (2, [FAKE16, FAKE16], [FAKE16, None], [1, 1], 1, 0, -1),          # null Y in entry 1
    (2, [FAKE16, FAKE16], [FAKE16, FAKE16], [1, -3], 1, 0, -1),       # N < 0
    (2, [FAKE16, FAKE16 + 8], [FAKE16, FAKE16], [1, 1], 1, 0, -4),    # W alignment
    (2, [FAKE16, FAKE16], [FAKE16, FAKE16 + 2], [1, 1], 1, 0, -4),    # Y alignment
    (3, [FAKE16] * 3, [FAKE16] * 3, [1] * 3, 9, 1, -3),               # GEMV path, M > 8
    (3, [FAKE16] * 3, [FAKE16] * 3, [1] * 3, 65, 3, -3),              # small-M path, M > 64
    (3, [FAKE16] * 3, [FAKE16] * 3, [1] * 3, 1, 5, -1),               # unknown path
    (2, [FAKE16, None], [FAKE16, None], [4, 0], 0, 0, 0),             # M = 0: empty
    (2, [None, None], [None, None], [0, 0], 3, 0, 0),                 # all N = 0: empty
])
def test_group_validation(L, count, Ws, Ys, Ns, M, path, status):
    n = max(len(Ws), 1)
    P = ctypes.c_void_p
    wa, ya = (P * n)(*Ws), (P * n)(*Ys)
    na = (ctypes.c_int64 * n)(*Ns)
    assert L.gemmq_gemm_group(12, count, wa, ya, na, FAKE16, M, 256, path, None) == status


def test_group_null_arrays(L):
    P = ctypes.c_void_p
    one_p, one_n = (P * 1)(FAKE16), (ctypes.c_int64 * 1)(1)
    assert L.gemmq_gemm_group(12, 1, None, one_p, one_n, FAKE16, 1, 256, 0, None) == -1
    assert L.gemmq_gemm_group(12, 1, one_p, None, one_n, FAKE16, 1, 256, 0, None) == -1
    assert L.gemmq_gemm_group(12, 1, one_p, one_p, None, FAKE16, 1, 256, 0, None) == -1
    assert L.gemmq_gemm_group(15, 1, one_p, one_p, one_n, FAKE16, 1, 256, 0, None) == -2
    assert L.gemmq_gemm_group(12, 1, one_p, one_p, one_n, None, 1, 256, 0, None) == -1


@pytest.mark.parametrize("args,status", [
    ((15, FAKE16, FAKE16, FAKE16, FAKE16, 1, 1, 256), -2),      # unknown format
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, 1, 1, 300), -3),      # K % 256 != 0
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, -1, 1, 256), -1),     # M < 0
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, 1, -1, 256), -1),     # N < 0
    ((12, None, FAKE16, FAKE16, FAKE16, 1, 1, 256), -1),        # null W
    ((12, FAKE16, None, FAKE16, FAKE16, 1, 1, 256), -1),        # null X
    ((12, FAKE16, FAKE16, None, FAKE16, 1, 1, 256), -1),        # null Xq
    ((12, FAKE16, FAKE16, FAKE16, None, 1, 1, 256), -1),        # null Y
    ((12, FAKE16 + 4, FAKE16, FAKE16, FAKE16, 1, 1, 256), -4),  # q4_K weights need 16 B
    ((12, FAKE16, FAKE16 + 4, FAKE16, FAKE16, 1, 1, 256), -4),  # X needs 16 B
    ((12, FAKE16, FAKE16, FAKE16 + 2, FAKE16, 1, 1, 256), -4),  # Xq needs 4 B
    ((12, FAKE16, FAKE16, FAKE16, FAKE16 + 1, 1, 1, 256), -4),  # Y needs 4 B
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, 0, 5, 256), 0),       # M = 0: empty
])
def test_linear_validation(L, args, status):
    fmt, W, X, Xq, Y, M, N, K = args
    assert L.gemmq_linear(fmt, W, X, Xq, Y, M, N, K, None) == status
    P = ctypes.c_void_p
    wa, ya, na = (P * 1)(W), (P * 1)(Y), (ctypes.c_int64 * 1)(N)
    for path in (0, 1):
        assert L.gemmq_linear_group(fmt, 1, wa, ya, na, X, Xq, M, K, path, None) == status


@pytest.mark.parametrize("args,status", [
    ((15, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 1, 1, 256, 0), -2),      # unknown format
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 1, 1, 300, 0), -3),      # K % 256 != 0
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, -1, 1, 256, 0), -1),     # M < 0
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 1, -1, 256, 0), -1),     # N < 0
    ((12, None, FAKE16, FAKE16, FAKE16, FAKE16, 1, 1, 256, 0), -1),        # null gate
    ((12, FAKE16, None, FAKE16, FAKE16, FAKE16, 1, 1, 256, 0), -1),        # null up
    ((12, FAKE16, FAKE16, None, FAKE16, FAKE16, 1, 1, 256, 0), -1),        # null X
    ((12, FAKE16, FAKE16, FAKE16, None, FAKE16, 1, 1, 256, 0), -1),        # null Xq
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, None, 1, 1, 256, 0), -1),        # null Y
    ((12, FAKE16, FAKE16 + 8, FAKE16, FAKE16, FAKE16, 1, 1, 256, 0), -4),  # up alignment
    ((12, FAKE16, FAKE16, FAKE16 + 4, FAKE16, FAKE16, 1, 1, 256, 0), -4),  # X alignment
    ((12, FAKE16, FAKE16, FAKE16, FAKE16 + 2, FAKE16, 1, 1, 256, 0), -4),  # Xq alignment
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16 + 1, 1, 1, 256, 0), -4),  # Y alignment
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 9, 1, 256, 1), -3),      # GEMV path, M > 8
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 1, 1, 256, 4), -1),      # unknown path
    ((13, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 4, 1, 256, 3), -2),      # small-M path: q4_K, q6_K
    ((14, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 17, 1, 256, 3), -3),     # small-M q6_K, M > 16
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 65, 1, 256, 3), -3),     # small-M path, M > 64
    ((12, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, 0, 5, 256, 0), 0),       # M = 0: empty
])
def test_linear_silu_mul_validation(L, args, status):
    assert L.gemmq_linear_silu_mul(*args, None) == status


@pytest.mark.parametrize("fmt", [12, 14, 10])
def test_linear_refused_before_the_quantizer(L, fmt):
    # a matmul that cannot be launched (M past the GEMM's grid) is refused before
    # the quantizer is enqueued: the call returns the shape error while X and Xq
    # are still untouched (no device is needed to reach this status: the check
    # precedes the device check, and nothing with these pointers is enqueued)
    P = ctypes.c_void_p
    wa, ya, na = (P * 1)(FAKE16), (P * 1)(FAKE16), (ctypes.c_int64 * 1)(1)
    M = gq.GEMM_MAX_M + 1
    for path in (0, 2):
        assert L.gemmq_linear_group(fmt, 1, wa, ya, na, FAKE16, FAKE16, M, 256, path, None) == -3
        assert L.gemmq_linear_silu_mul(fmt, FAKE16, FAKE16, FAKE16, FAKE16, FAKE16, M, 1, 256,
                                       path, None) == -3
    # with no matrix rows the call only quantizes, and that has no such limit
    na0 = (ctypes.c_int64 * 1)(0)
    assert L.gemmq_linear_group(fmt, 1, wa, ya, na0, FAKE16, FAKE16, M, 256, 0, None) == -5


def test_linear_group_arrays_and_paths(L):
    P = ctypes.c_void_p
    one_p, one_n = (P * 1)(FAKE16), (ctypes.c_int64 * 1)(1)
    args = (FAKE16, FAKE16, 1, 256)
    assert L.gemmq_linear_group(12, 0, one_p, one_p, one_n, *args, 0, None) == -1
    assert L.gemmq_linear_group(12, 5, one_p, one_p, one_n, *args, 0, None) == -1
    assert L.gemmq_linear_group(12, 1, None, one_p, one_n, *args, 0, None) == -1
    assert L.gemmq_linear_group(12, 1, one_p, None, one_n, *args, 0, None) == -1
    assert L.gemmq_linear_group(12, 1, one_p, one_p, None, *args, 0, None) == -1
    assert L.gemmq_linear_group(12, 1, one_p, one_p, one_n, *args, 4, None) == -1
    assert L.gemmq_linear_group(13, 1, one_p, one_p, one_n, *args, 3, None) == -2
    assert L.gemmq_linear_group(12, 1, one_p, one_p, one_n, FAKE16, FAKE16, 65, 256, 3,
                                None) == -3
    assert L.gemmq_linear_group(12, 1, one_p, one_p, one_n, FAKE16, FAKE16, 9, 256, 1,
                                None) == -3


@pytest.mark.parametrize("args,status", [
    ((FAKE16, FAKE16, -1, 256), -1),
    ((FAKE16, FAKE16, 1, 255), -3),
    ((FAKE16, FAKE16, 1, 0), -3),
    ((None, FAKE16, 1, 256), -1),
    ((FAKE16, None, 1, 256), -1),
    ((FAKE16 + 4, FAKE16, 1, 256), -4),   # X needs 16 B
    ((FAKE16, FAKE16 + 1, 1, 256), -4),   # Xq needs 4 B
    ((None, None, 0, 256), 0),            # M = 0: empty
])
def test_quantize_validation(L, args, status):
    X, Xq, M, K = args
    assert L.gemmq_quantize_q8K(X, Xq, M, K, None) == status


@pytest.mark.parametrize("args,status", [
    ((99, FAKE16, FAKE16, 1, 256), -2),
    ((12, FAKE16, FAKE16, 1, 512 + 3), -3),
    ((12, None, FAKE16, 1, 256), -1),
    ((12, FAKE16, None, 1, 256), -1),
    ((12, FAKE16, FAKE16 + 4, 1, 256), -4),  # Wf needs 16 B
    ((12, FAKE16, FAKE16, 0, 256), 0),
])
def test_decode_validation(L, args, status):
    assert L.gemmq_decode(*args, None) == status


def test_binding_checks_out_sizes(L):
    # the torch wrappers refuse an undersized output before any launch (no GPU
    # here: fake device tensors are never handed to the library)
    class FakeDev:
        is_cuda = True

        def __init__(self, n, dtype):
            import torch
            self.dtype, self._n = dtype, n
            self.shape = (n,)

        def numel(self):
            return self._n

        def is_contiguous(self):
            return True

        def data_ptr(self):
            raise AssertionError("reached the library")

    import torch
    w = FakeDev(144 * 4, torch.uint8)
    with pytest.raises(ValueError):
        gq.decode(12, w, 2, 512, out=FakeDev(2 * 512 - 1, torch.float32))


def test_binding_raises_named_error(L):
    with pytest.raises(gq.GemmqError) as e:
        gq._lib._check(-2, "gemmq_gemm")
    assert "UNSUPPORTED_FORMAT" in str(e.value)


def test_product_path_never_imports_oracle():
    # the product package and its binding must not reach the CPU oracle
    pkg = os.path.join(ROOT, "quant_packed_weight_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"import\s+oracle|from\s+oracle|liboracle|oracle[./]", text), f


@pytest.mark.parametrize("args,status", [
    ((12, FAKE16, FAKE16 * 4, 1, 256), -2),          # q4_K has no repacked layout
    ((256 + 14, FAKE16, FAKE16 * 4, 1, 256), -2),    # already repacked
    ((14, FAKE16, FAKE16 * 4, 1, 300), -3),          # K % 256 != 0
    ((14, FAKE16, FAKE16 * 4, -1, 256), -1),         # N < 0
    ((14, None, FAKE16 * 4, 1, 256), -1),            # null W
    ((14, FAKE16, None, 1, 256), -1),                # null Wr
    ((14, FAKE16 + 2, FAKE16 * 4, 1, 256), -4),      # W not 4-byte aligned
    ((14, FAKE16, FAKE16 * 4 + 4, 1, 256), -4),      # Wr not 16-byte aligned
    ((14, FAKE16, FAKE16 + 16, 1, 256), -1),         # overlapping buffers
    ((11, FAKE16, FAKE16 * 4, 0, 256), 0),           # N = 0: empty
])
def test_repack_validation(L, args, status):
    assert L.gemmq_repack(*args, None) == status


def test_repacked_formats_accepted_except_decode(L):
    # a repacked format validates like any weight format (16-byte aligned base)
    # and is refused only by the diagnostic decode
    assert L.gemmq_gemm(256 + 14, FAKE16 + 4, FAKE16, FAKE16, 1, 1, 256, None) == -4
    assert L.gemmq_gemm(256 + 11, FAKE16, FAKE16, FAKE16, 1, 1, 300, None) == -3
    assert L.gemmq_decode(256 + 14, FAKE16, FAKE16, 1, 256, None) == -2


@pytest.mark.parametrize("args,status", [
    ((0, 1, FAKE16, FAKE16), -1),        # iters < 1
    ((1, 0, FAKE16, FAKE16), -1),        # no workgroups
    ((1, 65536, FAKE16, FAKE16), -1),    # too many workgroups
    ((1, 1, None, FAKE16), -1),
    ((1, 1, FAKE16, None), -1),
    ((1, 1, FAKE16 + 2, FAKE16), -4),    # out needs 4 B
    ((1, 1, FAKE16, FAKE16 + 4), -4),    # clocks need 8 B
    ((gq.PROBE_MAX_ITERS + 1, 1, FAKE16, FAKE16), -1),  # past the iteration cap
])
def test_probe_validation(L, args, status):
    assert L.gemmq_probe_mfma_i8(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((1, 1, 3, FAKE16, FAKE16), -1),      # vector work per MFMA not in {0, 4, 8, 12, 16}
    ((1, 1, 20, FAKE16, FAKE16), -1),
    ((1, 1, -4, FAKE16, FAKE16), -1),
    ((0, 1, 8, FAKE16, FAKE16), -1),      # iters < 1
    ((1, 65536, 8, FAKE16, FAKE16), -1),  # too many workgroups
    ((1, 1, 8, None, FAKE16), -1),
    ((1, 1, 8, FAKE16, None), -1),
    ((1, 1, 8, FAKE16 + 2, FAKE16), -4),  # out needs 4 B
    ((1, 1, 8, FAKE16, FAKE16 + 4), -4),  # clocks need 8 B
    ((gq.PROBE_MAX_ITERS + 1, 1, 8, FAKE16, FAKE16), -1),
])
def test_probe_mfma_valu_validation(L, args, status):
    assert L.gemmq_probe_mfma_valu(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, 1024, FAKE16), -1),
    ((FAKE16, 1024, None), -1),
    ((FAKE16, 0, FAKE16), -1),            # nothing to read
    ((FAKE16, 1000, FAKE16), -1),         # not a multiple of 16
    ((FAKE16, (1 << 40) + 16, FAKE16), -1),
    ((FAKE16 + 8, 1024, FAKE16), -4),     # src needs 16 B
    ((FAKE16, 1024, FAKE16 + 2), -4),     # out needs 4 B
])
def test_probe_read_validation(L, args, status):
    assert L.gemmq_probe_read(*args, None) == status
