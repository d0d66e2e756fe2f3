"""GPU parity of the fp8 path: OCP E4M3 inputs (one byte each), fp32
accumulation in v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales), fp32 or bf16
output, against the fp64 oracle.  The operands move through the same LDS
machinery as the 16-bit path: 16-byte direct-to-LDS loads, XOR-swizzled
tiles, ds_read_b128 for K-contiguous and ds_read_b64_tr_b8 for
MN-contiguous operands ("Lds Optimization", "MFMA Transpose Load from LDS
(gfx950 only)").

Integer-valued inputs in {-2..2} are exact in E4M3 and every partial sum is
exact in fp32, so those results are unique and checked bit for bit; real
inputs use the tolerances of the 16-bit path (fp32 out: 1e-5*K; bf16 out:
2^-8*|ref| + 1e-5*K)."""
import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
import synth
import gpu_harness as H
from test_gpu_parity import every_tile_check

pytestmark = pytest.mark.gpu

ALL_LAYOUTS = [("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")]
FP8 = [lsm.GEMM_E4M3_F32, lsm.GEMM_E4M3_BF16]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.handle()


def check_full(M, N, K, la, lb, gdtype, dist, seeds, ldc_pad=0, extra_rows=0):
    print("CASE fp8", M, N, K, la, lb, gdtype, dist, seeds, flush=True)
    p = H.problem(M, N, K, synth.E4M3, la, lb, dist, seeds)
    C = H.run_gpu(p, gdtype, ldc=N + ldc_pad, extra_rows=extra_rows)
    H.assert_canary(C, M, N, gdtype)
    ref = H.oracle_full(p)
    if dist == "int":
        H.assert_exact(C[:M, :N], ref, gdtype, f"fp8 {M}x{N}x{K} {la}{lb}")
    else:
        H.assert_close(C[:M, :N], ref, K, gdtype, f"fp8 {M}x{N}x{K} {la}{lb}")


# Contiguous extents are multiples of 16 elements (16 bytes); everything else
# is ragged against the tiles.  One shape per kernel: 64 x 64 tile, 128 x 128
# tile (>= 256 tiles of 128), M <= 32 split-K ring.
SHAPES = [(272, 336, 208), (96, 160, 16), (2064, 2064, 144), (32, 1008, 1040), (16, 272, 4112)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gdtype", FP8)
def test_fp8_integer_exact(shape, la, lb, gdtype):
    M, N, K = shape
    check_full(M, N, K, la, lb, gdtype, "int", (121, 122), ldc_pad=3, extra_rows=1)


@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gdtype", FP8)
def test_fp8_real(la, lb, gdtype):
    check_full(304, 288, 528, la, lb, gdtype, "normal", (123, 124), ldc_pad=1, extra_rows=1)


@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_fp8_pingpong_ragged_integer_exact(la, lb):
    # >= 256 tiles of 256: the ping-pong kernel, ragged M and N edges
    M, N, K = 4112, 4096, 160
    print("CASE fp8 pingpong", M, N, K, la, lb, flush=True)
    p = H.problem(M, N, K, synth.E4M3, la, lb, "int", (125, 126))
    for gdtype, ldc in ((lsm.GEMM_E4M3_F32, N + 3), (lsm.GEMM_E4M3_BF16, N)):
        C = H.run_gpu(p, gdtype, ldc=ldc, extra_rows=1)
        H.assert_canary(C, M, N, gdtype)
        for r0, r1 in ((0, 2), (4095, 4097), (M - 2, M)):
            H.assert_exact(C[r0:r1, :N], H.oracle_rows(p, r0, r1), gdtype, f"rows {r0}")
        rng = np.random.default_rng(2)
        rows, cols = rng.integers(0, M, 4000), rng.integers(0, N, 4000)
        H.assert_exact(C[rows, cols], H.oracle_entries(p, rows, cols), gdtype, "entries")


def test_fp8_workload_8192_nn_f32():
    w = synth.WORKLOADS["e4m3_8192_nn_f32"]
    print("CASE fp8 8192", flush=True)
    p = H.problem(8192, 8192, 8192, synth.E4M3, "K", "MN", w["dist"], w["seeds"])
    C = H.run_gpu(p, lsm.GEMM_E4M3_F32)
    for r0, r1 in ((0, 2), (8191, 8192)):
        H.assert_close(C[r0:r1], H.oracle_rows(p, r0, r1), 8192, lsm.GEMM_E4M3_F32, f"rows {r0}")
    rng = np.random.default_rng(3)
    rows, cols = rng.integers(0, 8192, 2000), rng.integers(0, 8192, 2000)
    H.assert_close(C[rows, cols], H.oracle_entries(p, rows, cols), 8192, lsm.GEMM_E4M3_F32,
                   "entries")
    # a full row in every tile row and a full column in every tile column:
    # every 256 x 256 tile of the launch has checked entries
    every_tile_check(p, C, lsm.GEMM_E4M3_F32, False, seed=7)


def test_fp8_workload_8192_integer_exact_every_tile():
    # the workload's integer variant (values -2..2, exact in E4M3 and in the
    # fp32 sums): the unique result, bit for bit, in every tile
    print("CASE fp8 8192 int", flush=True)
    p = H.problem(8192, 8192, 8192, synth.E4M3, "K", "MN", "int", (6001, 6002))
    C = H.run_gpu(p, lsm.GEMM_E4M3_F32)
    every_tile_check(p, C, lsm.GEMM_E4M3_F32, True, seed=8)


def test_fp8_k_zero_writes_zeros():
    p = H.problem(64, 80, 0, synth.E4M3, "K", "MN", "int")
    C = H.run_gpu(p, lsm.GEMM_E4M3_F32, ldc=96, extra_rows=1)
    assert np.all(C[:64, :80] == 0)
    H.assert_canary(C, 64, 80, lsm.GEMM_E4M3_F32)


def test_fp8_unsupported_extents_rejected_untouched():
    # contiguous extents that are not whole 16-byte chunks: explicit
    # GEMM_ERR_UNSUPPORTED, nothing enqueued, C untouched
    h = H.handle()
    A = torch.zeros(1 << 16, dtype=torch.int8, device="cuda")
    B = torch.zeros(1 << 16, dtype=torch.int8, device="cuda")
    C = torch.full((4096,), 7.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    run = lambda M, N, K, lda, ldb, la, lb: lsm.gemm_run(h, A, B, C, M, N, K, lda, ldb, N, la, lb,
                                                         lsm.GEMM_E4M3_F32, s)
    assert run(16, 16, 24, 32, 16, 0, 1) == lsm.GEMM_ERR_UNSUPPORTED   # K % 16 (A K-contig)
    assert run(16, 24, 32, 32, 32, 0, 1) == lsm.GEMM_ERR_UNSUPPORTED   # N % 16 (B N-contig)
    assert run(24, 16, 32, 32, 32, 1, 0) == lsm.GEMM_ERR_UNSUPPORTED   # M % 16 (A M-contig)
    assert run(16, 16, 32, 40, 16, 0, 1) == lsm.GEMM_ERR_UNSUPPORTED   # lda not 16 bytes
    torch.cuda.synchronize()
    assert bool(torch.all(C == 7.0))


def test_fp8_footprint_beyond_2gib_rejected_untouched():
    # fp8 runs only on the direct-to-LDS kernels, whose buffer offsets are
    # 32-bit: an A footprint past 2^31 bytes is GEMM_ERR_UNSUPPORTED, with
    # nothing enqueued and C untouched.
    h = H.handle()
    M, N, K = 72, 64, 64
    lda = 1 << 25                           # 71 rows of 32 MiB: 2.2 GiB footprint
    assert ((M - 1) * lda + K) > (1 << 31)
    A = torch.zeros((M - 1) * lda + K, dtype=torch.int8, device="cuda")
    B = torch.zeros(K * N, dtype=torch.int8, device="cuda")
    C = torch.full((M * N,), 7.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    st = lsm.gemm_run(h, A, B, C, M, N, K, lda, N, N, lsm.GEMM_K_CONTIG, lsm.GEMM_MN_CONTIG,
                      lsm.GEMM_E4M3_F32, s)
    assert st == lsm.GEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool(torch.all(C == 7.0))
    del A
