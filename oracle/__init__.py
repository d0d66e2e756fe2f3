"""The oracle: a plain fp64 CPU GEMM (C, OpenMP) and its ctypes wrapper.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  The HIP library never calls it and
it never calls the HIP library; the two share no code.

C = A*B, C[m][n] = sum_k a(m,k) b(k,n) in fp64, loop order m -> k -> n
("An educational GEMM ladder for Helios GPUs", section "Educational GEMM
Ladder", problem statement C = AB; "Level 0 APIs" table: FP32 accumulation of
BF16 products, converted on store).  Layout 0 = K-contiguous, 1 =
MN-contiguous; dtype 0 = bf16, 1 = fp16 (two bytes per element), 2 = OCP
fp8 E4M3 (one byte per element, decode only); leading dimensions count
elements.
"""
import ctypes
import os

import numpy as np

BF16, F16, E4M3 = 0, 1, 2
K_CONTIG, MN_CONTIG = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_anyp = ctypes.c_void_p
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_f16.restype = ctypes.c_double
    lib.oracle_encode_bf16.argtypes = [ctypes.c_double]
    lib.oracle_encode_bf16.restype = ctypes.c_uint16
    lib.oracle_encode_f16.argtypes = [ctypes.c_double]
    lib.oracle_encode_f16.restype = ctypes.c_uint16
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e4m3.restype = ctypes.c_double
    lib.oracle_decode_array.argtypes = [_anyp, _f64p, _i64, _int]
    lib.oracle_decode_array.restype = None
    lib.oracle_encode_array.argtypes = [_f64p, _u16p, _i64, _int]
    lib.oracle_encode_array.restype = None
    lib.oracle_gemm_rows.argtypes = [_anyp, _anyp, _f64p, _i64, _i64, _i64, _i64, _i64,
                                     _i64, _int, _int, _int, _i64, _i64, _int]
    lib.oracle_gemm_rows.restype = _int
    lib.oracle_gemm.argtypes = [_anyp, _anyp, _f64p, _i64, _i64, _i64, _i64, _i64, _i64,
                                _int, _int, _int, _int]
    lib.oracle_gemm.restype = _int
    lib.oracle_gemm_entries.argtypes = [_anyp, _anyp, _i64, _i64, _i64, _i64, _i64, _int,
                                        _int, _int, _i64p, _i64p, _i64, _f64p, _int]
    lib.oracle_gemm_entries.restype = _int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = _int
    _lib = lib
    return lib


def _u16(x):
    return np.ascontiguousarray(np.asarray(x).reshape(-1).view(np.uint16))


def _elements(x, dtype):
    """Contiguous storage of an element array: uint8 for e4m3, uint16 else."""
    a = np.asarray(x).reshape(-1)
    return np.ascontiguousarray(a.view(np.uint8) if dtype == E4M3 else a.view(np.uint16))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def decode(bits, dtype):
    """Exact fp64 values of bf16/fp16 (uint16) or e4m3 (uint8) bit patterns."""
    b = _elements(bits, dtype)
    out = np.empty(b.size, dtype=np.float64)
    _load().oracle_decode_array(_ptr(b), out, b.size, dtype)
    return out.reshape(np.shape(bits))


def encode(x, dtype):
    """Round-to-nearest-even of fp64 values to bf16/fp16 bit patterns."""
    v = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1))
    out = np.empty(v.size, dtype=np.uint16)
    _load().oracle_encode_array(v, out, v.size, dtype)
    return out.reshape(np.shape(x))


def gemm(A, B, M, N, K, lda, ldb, layoutA, layoutB, dtype, threads=0):
    """Full C (M x N, fp64, row-major) from flat bf16/fp16 storage A and B."""
    C = np.empty((M, N), dtype=np.float64)
    a, b = _elements(A, dtype), _elements(B, dtype)
    rc = _load().oracle_gemm(_ptr(a), _ptr(b), C.reshape(-1) if C.size else np.empty(1),
                             M, N, K, lda, ldb, max(N, 1), layoutA, layoutB, dtype, threads)
    if rc:
        raise ValueError("oracle_gemm: invalid arguments")
    return C


def gemm_rows(A, B, M, N, K, lda, ldb, layoutA, layoutB, dtype, row_begin, row_end,
              threads=0):
    """Rows [row_begin, row_end) of C."""
    C = np.empty((row_end - row_begin, N), dtype=np.float64)
    a, b = _elements(A, dtype), _elements(B, dtype)
    rc = _load().oracle_gemm_rows(_ptr(a), _ptr(b), C.reshape(-1) if C.size else np.empty(1),
                                  M, N, K, lda, ldb, max(N, 1), layoutA, layoutB, dtype,
                                  row_begin, row_end, threads)
    if rc:
        raise ValueError("oracle_gemm_rows: invalid arguments")
    return C


def gemm_entries(A, B, M, N, K, lda, ldb, layoutA, layoutB, dtype, rows, cols, threads=0):
    """C[rows[i], cols[i]] for each i."""
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    c = np.ascontiguousarray(np.asarray(cols, dtype=np.int64).reshape(-1))
    out = np.empty(r.size, dtype=np.float64)
    a, b = _elements(A, dtype), _elements(B, dtype)
    rc = _load().oracle_gemm_entries(_ptr(a), _ptr(b), M, N, K, lda, ldb, layoutA, layoutB,
                                     dtype, r, c, r.size, out, threads)
    if rc:
        raise ValueError("oracle_gemm_entries: invalid arguments")
    return out


def max_threads():
    return _load().oracle_max_threads()
