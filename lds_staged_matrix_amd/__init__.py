"""Python binding of the LDS-staged GEMM C ABI (include/lds_gemm.h).

Argument marshalling only: every step of C <- A*B runs in the HIP library
liblds_gemm.so built in this directory.  There is no fallback: if the
library is missing, every entry point raises.

Names mirror the C ABI: gemm_create, gemm_run, gemm_destroy, gemm_status_str.
Pointers may be passed as integers or as objects with a ``data_ptr()`` method
(torch tensors); streams as integers, objects with a ``cuda_stream``
attribute (torch streams) or None for the null stream.
"""
import ctypes
import os

__all__ = [
    "GEMM_K_CONTIG", "GEMM_MN_CONTIG",
    "GEMM_BF16_F32", "GEMM_BF16_BF16", "GEMM_F16_F16", "GEMM_F16_F32", "GEMM_E4M3_F32",
    "GEMM_E4M3_BF16",
    "GEMM_OK", "GEMM_ERR_INVALID_ARG", "GEMM_ERR_UNSUPPORTED", "GEMM_ERR_DEVICE",
    "GEMM_ERR_LAUNCH", "GemmError", "library_path", "load_library", "gemm_create",
    "gemm_run", "gemm_destroy", "gemm_status_str", "EXPORTED_SYMBOLS", "Library",
    "ablation_library",
]

GEMM_K_CONTIG, GEMM_MN_CONTIG = 0, 1
GEMM_BF16_F32, GEMM_BF16_BF16, GEMM_F16_F16, GEMM_F16_F32 = 0, 1, 2, 3
GEMM_E4M3_F32, GEMM_E4M3_BF16 = 4, 5
GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED, GEMM_ERR_DEVICE, GEMM_ERR_LAUNCH = range(5)
EXPORTED_SYMBOLS = ("gemm_create", "gemm_run", "gemm_destroy", "gemm_status_str")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "liblds_gemm.so"
_lib = None


class GemmError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {gemm_status_str(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with lds_staged_matrix_amd/build.py "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.gemm_create.argtypes = [ctypes.POINTER(vp)]
    lib.gemm_create.restype = i32
    lib.gemm_run.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, i32, vp]
    lib.gemm_run.restype = i32
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_destroy.restype = i32
    lib.gemm_status_str.argtypes = [i32]
    lib.gemm_status_str.restype = ctypes.c_char_p
    return lib


def load_library():
    """Load liblds_gemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _open(library_path())
    return _lib


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _int(x, bits, name):
    """x as a Python int that fits the C ABI's signed `bits`-bit parameter.
    ctypes would silently keep only the low bits of a larger value."""
    v = int(x)
    if not -(1 << (bits - 1)) <= v < (1 << (bits - 1)):
        raise OverflowError(f"{name}={v} does not fit the C ABI's int{bits}_t parameter")
    return v


def _sizes(M, N, K, lda, ldb, ldc, layoutA, layoutB, dtype):
    return ([_int(v, 64, n) for v, n in zip((M, N, K, lda, ldb, ldc),
                                             ("M", "N", "K", "lda", "ldb", "ldc"))] +
            [_int(v, 32, n) for v, n in zip((layoutA, layoutB, dtype),
                                             ("layoutA", "layoutB", "dtype"))])


def _stream(s):
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def gemm_create():
    """Create a handle on the current device; raises GemmError on failure."""
    h = ctypes.c_void_p()
    st = load_library().gemm_create(ctypes.byref(h))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_create")
    return h


def gemm_run(h, A, B, C, M, N, K, lda, ldb, ldc, layoutA, layoutB, dtype, stream=None) -> int:
    """Enqueue C <- A*B; returns the gemm_status code (0 on success)."""
    return load_library().gemm_run(h, _ptr(A), _ptr(B), _ptr(C),
                                   *_sizes(M, N, K, lda, ldb, ldc, layoutA, layoutB, dtype),
                                   _stream(stream))


def gemm_destroy(h) -> int:
    return load_library().gemm_destroy(h)


def gemm_status_str(status: int) -> str:
    return load_library().gemm_status_str(_int(status, 32, "status")).decode()


class Library:
    """The same four entry points bound to one specific build of the library
    (the default build, or an A/B build from ablation_library())."""

    def __init__(self, path):
        self.path = path
        self._lib = _open(path)

    def gemm_create(self):
        h = ctypes.c_void_p()
        st = self._lib.gemm_create(ctypes.byref(h))
        if st != GEMM_OK:
            raise GemmError(st, "gemm_create")
        return h

    def gemm_run(self, h, A, B, C, M, N, K, lda, ldb, ldc, layoutA, layoutB, dtype,
                 stream=None) -> int:
        return self._lib.gemm_run(h, _ptr(A), _ptr(B), _ptr(C),
                                  *_sizes(M, N, K, lda, ldb, ldc, layoutA, layoutB, dtype),
                                  _stream(stream))

    def gemm_destroy(self, h) -> int:
        return self._lib.gemm_destroy(h)

    def gemm_status_str(self, status: int) -> str:
        return self._lib.gemm_status_str(_int(status, 32, "status")).decode()


def ablation_library(name: str) -> Library:
    """An A/B build of the library that changes one design choice (names in
    build.VARIANTS); built by build.build_all().  Only benchmarks and tests
    use these."""
    from . import build as _build
    if name not in _build.VARIANTS:
        raise ValueError(f"unknown ablation build {name!r}; known: {sorted(_build.VARIANTS)}")
    return Library(_build.variant_path(name))
