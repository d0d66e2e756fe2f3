"""The 64 x 64 direct-to-LDS kernel with four LDS stages, against the oracle.

The dispatcher gives the 64 x 64 tile four LDS stages when the A and B panels
that one XCD's workgroups read over the whole K range exceed that XCD's 4 MiB
L2 (lds_layout.h, xcd_max_panel_bytes).  Every shape here is first checked to
take that path (the same rule, evaluated by the host build of lds_layout.h),
then compared with the oracle: integer inputs bit for bit in all four layouts
with canaries around C, real inputs within the output type's tolerance.
"""
import ctypes

import pytest

import lds_staged_matrix_amd as lsm
from lds_staged_matrix_amd import build as hip_build
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

ALL_LAYOUTS = [("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")]
L2_BYTES_PER_XCD = 4 << 20


def takes_four_stages(M, N, K, es):
    lib = ctypes.CDLL(hip_build.layout_host_path(""))
    lib.lsm_xcd_max_panel_bytes.restype = ctypes.c_longlong
    lib.lsm_xcd_max_panel_bytes.argtypes = [ctypes.c_int] * 3 + [ctypes.c_longlong] * 2
    t128 = -(-M // 128) * -(-N // 128)
    panel = 64 * K * es
    return (M > 32 and t128 < 256 and
            lib.lsm_xcd_max_panel_bytes(-(-M // 64), -(-N // 64), 8, panel, panel) > L2_BYTES_PER_XCD)


def check(M, N, K, la, lb, gdtype, dist, seeds, **kw):
    es = 1 if H.IN_OF[gdtype] == synth.E4M3 else 2
    assert takes_four_stages(M, N, K, es), "shape does not exercise the four-stage kernel"
    print(f"CASE four-stage {M}x{N}x{K} {la}{lb} dtype {gdtype} {dist}", flush=True)
    p = H.problem(M, N, K, H.IN_OF[gdtype], la, lb, dist, seeds, extra_pad=kw.get("extra_pad", 0))
    C = H.run_gpu(p, gdtype, ldc=N + kw.get("ldc_pad", 0), extra_rows=kw.get("extra_rows", 0))
    H.assert_canary(C, M, N, gdtype)
    ref = H.oracle_full(p)
    if dist == "int":
        H.assert_exact(C[:M, :N], ref, gdtype, f"{M}x{N}x{K} {la}{lb}")
    else:
        H.assert_close(C[:M, :N], ref, K, gdtype, f"{M}x{N}x{K} {la}{lb}")


# 8 x 8 tiles (one column of 8 tile rows per XCD), a K tail of 8, and
# ragged M or N in both orientations
SHAPES = [(512, 512, 4096), (500, 300, 6152), (200, 1000, 6152), (1000, 200, 6152)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_four_stage_integer_exact(shape, la, lb):
    M, N, K = shape
    check(M, N, K, la, lb, lsm.GEMM_BF16_F32, "int", (41, 42), extra_pad=1, ldc_pad=3,
          extra_rows=2)


@pytest.mark.parametrize("gdtype", [lsm.GEMM_BF16_BF16, lsm.GEMM_F16_F16, lsm.GEMM_F16_F32])
def test_four_stage_real(gdtype):
    check(500, 300, 6152, "K", "MN", gdtype, "normal", (43, 44), ldc_pad=5, extra_rows=1)


@pytest.mark.parametrize("shape", [(512, 512, 8192), (496, 304, 12304)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gdtype", [lsm.GEMM_E4M3_F32, lsm.GEMM_E4M3_BF16])
def test_four_stage_fp8_integer_exact(shape, la, lb, gdtype):
    M, N, K = shape
    check(M, N, K, la, lb, gdtype, "int", (45, 46), ldc_pad=16, extra_rows=1)


def test_two_stages_below_the_l2():
    """The shapes just below the threshold keep the double buffer (and the
    1500 x 1152 x 896 workload is one of them)."""
    assert not takes_four_stages(512, 512, 3072, 2)
    assert not takes_four_stages(1024, 1024, 2048, 2)
    assert not takes_four_stages(1500, 1152, 896, 2)
    assert not takes_four_stages(256, 256, 256, 2)
