"""The A/B build of the ping-pong kernel on the 32 x 32 MFMAs (build variant
"mfma32": v_mfma_f32_32x32x16 for 16-bit and v_mfma_scale_f32_32x32x64_f8f6f4
for E4M3 inputs), against the library (v_mfma_f32_16x16x32 and
v_mfma_scale_f32_16x16x128_f8f6f4) and the oracle.

The build changes only the MFMA shape of the ping-pong kernel: its
LDS layout of MN-contiguous tiles (the transposed-read swizzle of each
fragment shape), fragment reads, accumulator layout and both epilogues (the
LDS-staged one, taken when C rows are 16-byte aligned, and the direct one).
On integer inputs the result is unique, so the two must agree bit for bit;
the library's own output is checked against the oracle on sampled rows.
"""
import numpy as np
import pytest

import lds_staged_matrix_amd as lsm
import gpu_harness as H

pytestmark = pytest.mark.gpu

ALL_LAYOUTS = [("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")]
DTYPES = [lsm.GEMM_BF16_F32, lsm.GEMM_BF16_BF16, lsm.GEMM_F16_F16, lsm.GEMM_F16_F32]
# 4104 x 4088: 17 x 16 tiles of 256 (at least 256, so the ping-pong kernel),
# ragged in M and N but whole 16-byte chunks along every contiguous extent
# (else the register-staged kernel serves the shape); K = 264 ends in a
# partial K tile of 8.
M, N, K = 4104, 4088, 264
# ldc 4096: rows 16-byte aligned for every output type (LDS-staged epilogue);
# ldc 4090: not aligned for any (direct epilogue).
LDCS = [4096, 4090]
ROWS = [0, 1, 255, 256, 2047, 4095, 4096, 4103]


def takes_pingpong(M, N, K):
    """The dispatch rule for 16-bit inputs: M > 32, at least 256 tiles of
    256 x 256, and every contiguous extent a whole number of 16-byte chunks
    (the 32-bit offset limit is far away at these sizes)."""
    tiles = -(-M // 256) * -(-N // 256)
    return M > 32 and tiles >= 256 and all((2 * x) % 16 == 0 for x in (M, N, K))


def test_shape_takes_the_pingpong_kernel():
    assert takes_pingpong(M, N, K)
    assert not takes_pingpong(4100, 4090, 264)   # ragged chunks: register-staged kernel


@pytest.fixture(scope="module")
def variant():
    lib = lsm.ablation_library("mfma32")
    h = lib.gemm_create()
    yield lib, h
    lib.gemm_destroy(h)


@pytest.mark.parametrize("gd", DTYPES)
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_mfma32_build_matches_the_library(variant, gd, la, lb):
    p = H.problem(M, N, K, H.IN_OF[gd], la, lb, "int", (61, 62))
    want = H.oracle_entries(p, np.repeat(ROWS, N), np.tile(np.arange(N), len(ROWS)))
    want = want.reshape(len(ROWS), N)
    for ldc in LDCS:
        print(f"CASE mfma32 {M}x{N}x{K} {la}{lb} dtype {gd} ldc {ldc}", flush=True)
        lib_out = H.run_gpu(p, gd, ldc=ldc, extra_rows=1)
        H.assert_canary(lib_out, M, N, gd)
        H.assert_exact(lib_out[ROWS, :N], want, gd, f"library {la}{lb} ldc {ldc}")
        got = H.run_gpu(p, gd, ldc=ldc, extra_rows=1, lib=variant)
        H.assert_canary(got, M, N, gd)
        bad = np.count_nonzero(got != lib_out)
        assert bad == 0, f"mfma32 build differs from the library in {bad} entries ({la}{lb}, ldc {ldc})"


# E4M3: every extent a multiple of 16 bytes; K = 272 ends in a partial K tile
# of 16 (BK 128).
M8, N8, K8 = 4112, 4096, 272
DTYPES8 = [lsm.GEMM_E4M3_F32, lsm.GEMM_E4M3_BF16]


@pytest.mark.parametrize("gd", DTYPES8)
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_mfma32_build_matches_the_library_fp8(variant, gd, la, lb):
    p = H.problem(M8, N8, K8, H.IN_OF[gd], la, lb, "int", (65, 66))
    rows = [0, 1, 255, 256, 2047, 4095, 4096, 4111]
    want = H.oracle_entries(p, np.repeat(rows, N8), np.tile(np.arange(N8), len(rows)))
    want = want.reshape(len(rows), N8)
    for ldc in (4096, 4097):   # C rows 16-byte aligned (LDS-staged epilogue) or not (direct)
        print(f"CASE mfma32 fp8 {M8}x{N8}x{K8} {la}{lb} dtype {gd} ldc {ldc}", flush=True)
        lib_out = H.run_gpu(p, gd, ldc=ldc, extra_rows=1)
        H.assert_canary(lib_out, M8, N8, gd)
        H.assert_exact(lib_out[rows, :N8], want, gd, f"library fp8 {la}{lb} ldc {ldc}")
        got = H.run_gpu(p, gd, ldc=ldc, extra_rows=1, lib=variant)
        H.assert_canary(got, M8, N8, gd)
        bad = np.count_nonzero(got != lib_out)
        assert bad == 0, f"mfma32 build differs from the library in {bad} entries (fp8 {la}{lb}, ldc {ldc})"


def test_mfma32_build_real_inputs(variant):
    """Real-valued operands: within the bf16-output tolerance of the oracle."""
    gd = lsm.GEMM_BF16_BF16
    print(f"CASE mfma32 real {M}x{N}x{K} NN bf16 out", flush=True)
    p = H.problem(M, N, K, H.IN_OF[gd], "K", "MN", "normal", (63, 64))
    got = H.run_gpu(p, gd, ldc=4096, lib=variant)
    ref = H.oracle_entries(p, np.repeat(ROWS, N), np.tile(np.arange(N), len(ROWS)))
    H.assert_close(got[ROWS, :N], ref.reshape(len(ROWS), N), K, gd, "mfma32 real")


@pytest.mark.parametrize("k", [0, 8, 64, 72, 128])
def test_mfma32_build_short_k(variant, k):
    """The ping-pong prologue's cases: no K tile (C = 0), one K tile (full or
    partial) and two (the second partial or full), against the library."""
    gd = lsm.GEMM_BF16_F32
    print(f"CASE mfma32 short K {M}x{N}x{k}", flush=True)
    p = H.problem(M, N, k, H.IN_OF[gd], "K", "MN", "int", (65, 66))
    lib_out = H.run_gpu(p, gd, ldc=4096)
    got = H.run_gpu(p, gd, ldc=4096, lib=variant)
    want = H.oracle_entries(p, np.repeat(ROWS, N), np.tile(np.arange(N), len(ROWS)))
    H.assert_exact(lib_out[ROWS, :N], want.reshape(len(ROWS), N), gd, f"library K={k}")
    assert np.count_nonzero(got != lib_out) == 0, f"mfma32 build differs from the library at K={k}"
