"""Every kernel instance the dispatcher can choose, against the oracle.

The library instantiates each kernel for every operand layout and element
type; which one runs depends on the shape class.  Here one shape per class
runs in all four layouts and with every output type.  On integer inputs the
result is unique: sampled rows (the first, the last and ones at tile edges)
and a random sample of entries must equal the oracle's bit for bit.  On real
inputs (uniform in [-1, 1]) they must lie within the output type's
tolerance.  C outside the M x N block must keep its canary.  Each shape is first
checked to fall in its class by the dispatch rule written out below.
"""
import ctypes

import numpy as np
import pytest

import lds_staged_matrix_amd as lsm
from lds_staged_matrix_amd import build as hip_build
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

ALL_LAYOUTS = [("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")]
DTYPES16 = [lsm.GEMM_BF16_F32, lsm.GEMM_BF16_BF16, lsm.GEMM_F16_F16, lsm.GEMM_F16_F32]
DTYPES8 = [lsm.GEMM_E4M3_F32, lsm.GEMM_E4M3_BF16]
L2_BYTES_PER_XCD = 4 << 20


def cdiv(a, b):
    return -(-a // b)


def shape_class(M, N, K, la, lb, es):
    """The kernel gemm_run picks: the rule of its dispatcher, restated."""
    a_inner = K if la == "K" else M
    b_inner = N if lb == "MN" else K
    dma = (a_inner * es) % 16 == 0 and (b_inner * es) % 16 == 0
    t256, t128 = cdiv(M, 256) * cdiv(N, 256), cdiv(M, 128) * cdiv(N, 128)
    if not dma:
        assert es == 2, "8-bit inputs need whole 16-byte chunks"
        if M <= 32:
            return "reg-skinny"
        return "reg-big" if t256 >= 256 else "reg-mid" if t128 >= 64 else "reg-small"
    if M <= 32:
        return "ring"
    if t256 >= 256:
        return "pingpong"
    if t128 >= 256:
        return "dma128"
    lib = ctypes.CDLL(hip_build.layout_host_path(""))
    lib.lsm_xcd_max_panel_bytes.restype = ctypes.c_longlong
    lib.lsm_xcd_max_panel_bytes.argtypes = [ctypes.c_int] * 3 + [ctypes.c_longlong] * 2
    panel = 64 * K * es
    over = lib.lsm_xcd_max_panel_bytes(cdiv(M, 64), cdiv(N, 64), 8, panel, panel) > L2_BYTES_PER_XCD
    return "dma64x4" if over else "dma64"


# (class, M, N, K) for 16-bit inputs: multiples of 8 reach the direct-to-LDS
# kernels, odd extents the register-staged ones
CASES16 = [
    ("pingpong", 4104, 4088, 72),      # 17 x 16 tiles of 256, two K tiles, the second partial
    ("dma128", 2056, 2048, 72),        # 17 x 16 tiles of 128
    ("dma64", 520, 264, 136),
    ("dma64x4", 512, 512, 4096),       # operand panels beyond one XCD's L2
    ("ring", 32, 1000, 1032),
    ("reg-big", 4097, 4089, 73),
    ("reg-mid", 1025, 1031, 73),
    ("reg-small", 130, 200, 73),
    ("reg-skinny", 17, 1001, 73),
]
# 8-bit inputs: every extent a multiple of 16
CASES8 = [
    ("pingpong", 4112, 4096, 144),
    ("dma128", 2064, 2048, 144),
    ("dma64", 528, 272, 160),
    ("dma64x4", 512, 512, 8192),
    ("ring", 32, 1024, 1040),
]


def check(cls, M, N, K, la, lb, gd, seed, dist, lib=None, what="every-kernel"):
    """One case against the oracle; `lib` = (Library, handle) runs an A/B build."""
    es = 1 if H.IN_OF[gd] == synth.E4M3 else 2
    assert shape_class(M, N, K, la, lb, es) == cls, (cls, M, N, K, la, lb)
    print(f"CASE {what} {cls} {M}x{N}x{K} {la}{lb} dtype {gd} {dist}", flush=True)
    p = H.problem(M, N, K, H.IN_OF[gd], la, lb, dist, (seed, seed + 1))
    C = H.run_gpu(p, gd, extra_rows=1, lib=lib)
    H.assert_canary(C, M, N, gd)
    rows = sorted({0, 1, min(M - 1, 63), min(M - 1, 64), M // 2, M - 2, M - 1})
    want = H.oracle_entries(p, np.repeat(rows, N), np.tile(np.arange(N), len(rows)))
    rng = np.random.default_rng(seed)
    r, c = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
    if dist == "int":
        H.assert_exact(C[rows, :N], want.reshape(len(rows), N), gd, f"{cls} {la}{lb} rows")
        H.assert_exact(C[r, c], H.oracle_entries(p, r, c), gd, f"{cls} {la}{lb} sample")
    else:
        H.assert_close(C[rows, :N], want.reshape(len(rows), N), K, gd, f"{cls} {la}{lb} rows")
        H.assert_close(C[r, c], H.oracle_entries(p, r, c), K, gd, f"{cls} {la}{lb} sample")


@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("case", CASES16, ids=lambda c: c[0])
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gd", DTYPES16)
def test_every_16bit_kernel(case, la, lb, gd, dist):
    cls, M, N, K = case
    check(cls, M, N, K, la, lb, gd, 700 + 10 * gd, dist)


@pytest.mark.parametrize("dist", ["int", "uniform"])
@pytest.mark.parametrize("case", CASES8, ids=lambda c: c[0])
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gd", DTYPES8)
def test_every_8bit_kernel(case, la, lb, gd, dist):
    cls, M, N, K = case
    check(cls, M, N, K, la, lb, gd, 800 + 10 * gd, dist)
