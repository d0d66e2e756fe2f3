"""GPU parity: the HIP GEMM through the C ABI against the fp64 oracle.

Every case prints its shape, layouts, dtype and seed before running, so a
failing case is named even if the process dies.
"""
import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

ALL_LAYOUTS = [("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")]
ALL_DTYPES = [lsm.GEMM_BF16_F32, lsm.GEMM_BF16_BF16, lsm.GEMM_F16_F16, lsm.GEMM_F16_F32]


def announce(*what):
    print("CASE", *what, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.handle()


def check_full(M, N, K, la, lb, gdtype, dist, seeds, scale=1.0, extra_pad=0, ldc_pad=0,
               extra_rows=0):
    announce(M, N, K, la, lb, gdtype, dist, seeds)
    p = H.problem(M, N, K, H.IN_OF[gdtype], la, lb, dist, seeds, scale, extra_pad)
    C = H.run_gpu(p, gdtype, ldc=N + ldc_pad, extra_rows=extra_rows)
    H.assert_canary(C, M, N, gdtype)
    ref = H.oracle_full(p)
    if dist == "int":
        H.assert_exact(C[:M, :N], ref, gdtype, f"{M}x{N}x{K} {la}{lb}")
    else:
        H.assert_close(C[:M, :N], ref, K, gdtype, f"{M}x{N}x{K} {la}{lb}")


# ------------------------------------------------------------------ small shapes

@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gdtype", ALL_DTYPES)
def test_256_cube_integer_exact(la, lb, gdtype):
    check_full(256, 256, 256, la, lb, gdtype, "int", (1001, 1002))


@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gdtype", ALL_DTYPES)
def test_256_cube_real(la, lb, gdtype):
    check_full(256, 256, 256, la, lb, gdtype, "uniform", (1001, 1002))


RAGGED = [(1, 1, 1), (31, 33, 17), (33, 31, 8), (63, 65, 64), (64, 64, 65),
          (255, 257, 100), (257, 255, 136), (129, 127, 200), (32, 200, 72), (5, 300, 129),
          (100, 96, 16), (96, 100, 48)]


@pytest.mark.parametrize("shape", RAGGED)
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_ragged_integer_exact(shape, la, lb):
    M, N, K = shape
    check_full(M, N, K, la, lb, lsm.GEMM_BF16_F32, "int", (7, 8), extra_pad=1, ldc_pad=3,
               extra_rows=2)


@pytest.mark.parametrize("shape", RAGGED[::2])
@pytest.mark.parametrize("gdtype", [lsm.GEMM_BF16_BF16, lsm.GEMM_F16_F16])
def test_ragged_real_16bit_out(shape, gdtype):
    M, N, K = shape
    check_full(M, N, K, "K", "MN", gdtype, "normal", (17, 18), ldc_pad=5, extra_rows=1)


@pytest.mark.parametrize("K", [16, 64, 128, 192, 8 * 3])
def test_k_step_counts(K):
    # prologue / epilogue with 1, 2 and 3 K steps and a partial step
    for la, lb in ALL_LAYOUTS:
        check_full(96, 160, K, la, lb, lsm.GEMM_BF16_F32, "int", (21, 22))


def test_k_zero_writes_zeros():
    announce("K=0")
    p = H.problem(70, 90, 0, synth.BF16, "K", "MN", "int")
    C = H.run_gpu(p, lsm.GEMM_BF16_F32, ldc=96, extra_rows=1)
    assert np.all(C[:70, :90] == 0)
    H.assert_canary(C, 70, 90, lsm.GEMM_BF16_F32)


def test_identity_and_permutation():
    announce("identity/permutation")
    rng = np.random.default_rng(4)
    K, N = 384, 320
    b = synth.quantize(synth.draw(41, K * N, "normal"), synth.BF16).reshape(K, N)
    ident = synth.quantize(np.eye(K), synth.BF16)
    perm = rng.permutation(K)
    P = synth.quantize(np.eye(K)[perm], synth.BF16)
    ones = synth.quantize(np.ones((K, K)), synth.BF16)
    bv = H.oracle.decode(b, H.oracle.BF16)
    for la, lb in ALL_LAYOUTS:
        for a, want in ((ident, bv), (P, bv[perm])):
            p = synth.layout_problem(a, b, synth.BF16, la, lb)
            C = H.run_gpu(p, lsm.GEMM_BF16_F32)
            assert np.array_equal(C.astype(np.float64), want)
        ob = synth.quantize(np.ones((K, N)), synth.BF16)
        C = H.run_gpu(synth.layout_problem(ones, ob, synth.BF16, la, lb), lsm.GEMM_BF16_F32)
        assert np.all(C == K)


def test_cross_layout_bit_identical():
    announce("cross-layout")
    a, b = synth.make_logical(300, 272, 264, synth.BF16, "uniform", 51, 52)
    outs = []
    for la, lb in ALL_LAYOUTS:
        pa = H.ld_pad(264 if la == "K" else 300)
        pb = H.ld_pad(272 if lb == "MN" else 264)
        p = synth.layout_problem(a, b, synth.BF16, la, lb, pa, pb)
        outs.append(H.run_gpu(p, lsm.GEMM_BF16_F32))
    # the MFMA k order is the same in every layout, so the fp32 sums agree bit for bit
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_deterministic():
    announce("determinism")
    p = H.problem(1000, 1000, 1000, synth.BF16, "K", "MN", "normal", (61, 62))
    c1 = H.run_gpu(p, lsm.GEMM_BF16_F32)
    c2 = H.run_gpu(p, lsm.GEMM_BF16_F32)
    assert np.array_equal(c1, c2)


# ------------------------------------------------------------------ workload shapes

def test_config_fp16_1500x1152x896_real():
    w = synth.WORKLOADS["f16_1500x1152x896_nn_f16"]
    check_full(1500, 1152, 896, "K", "MN", lsm.GEMM_F16_F16, "normal", w["seeds"], w["scale"])


def test_config_fp16_1500x1152x896_integer_exact():
    check_full(1500, 1152, 896, "K", "MN", lsm.GEMM_F16_F16, "int", (2001, 2002))


@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_big_tile_ragged_integer_exact(la, lb):
    # 17 x 16 tiles of 256: the 256 x 256 kernel, with ragged M, N and K edges
    M, N, K = 4133, 4077, 136
    announce(M, N, K, la, lb)
    p = H.problem(M, N, K, synth.BF16, la, lb, "int", (71, 72))
    C = H.run_gpu(p, lsm.GEMM_BF16_F32, ldc=N + 3, extra_rows=1)
    H.assert_canary(C, M, N, lsm.GEMM_BF16_F32)
    for r0, r1 in ((0, 9), (250, 262), (3838, 3842), (4090, 4133)):
        H.assert_exact(C[r0:r1, :N], H.oracle_rows(p, r0, r1), lsm.GEMM_BF16_F32, f"rows {r0}")
    rng = np.random.default_rng(0)
    rows, cols = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
    H.assert_exact(C[rows, cols], H.oracle_entries(p, rows, cols), lsm.GEMM_BF16_F32, "entries")


# The LDS-staged epilogue (16-byte C stores, used when C rows are 16-byte
# aligned): ragged M and N edges with ldc = N, every output type, on the
# 256 x 256 ping-pong kernel and the 128 x 128 kernel.
LDS_EPI = [(4100, 4104, 136), (2050, 2056, 264), (2048, 2052, 72)]


@pytest.mark.parametrize("shape", LDS_EPI)
@pytest.mark.parametrize("gdtype", ALL_DTYPES)
def test_lds_staged_epilogue_edges_integer_exact(shape, gdtype):
    M, N, K = shape
    for la, lb in (ALL_LAYOUTS if gdtype == lsm.GEMM_BF16_BF16 else ALL_LAYOUTS[:1]):
        announce("lds epilogue", M, N, K, la, lb, gdtype)
        p = H.problem(M, N, K, H.IN_OF[gdtype], la, lb, "int", (111, 112))
        C = H.run_gpu(p, gdtype, ldc=N, extra_rows=1)
        H.assert_canary(C, M, N, gdtype)
        rng = np.random.default_rng(1)
        for r0, r1 in ((0, 2), (M - 3, M)):
            H.assert_exact(C[r0:r1, :N], H.oracle_rows(p, r0, r1), gdtype, f"rows {r0}")
        cols = np.concatenate([np.arange(N - 40, N), rng.integers(0, N, 2000)])
        rows = rng.integers(0, M, cols.size)
        H.assert_exact(C[rows, cols], H.oracle_entries(p, rows, cols), gdtype, "entries")


@pytest.mark.parametrize("shape", [(4100, 4104, 136), (2050, 2056, 264)])
def test_c_base_not_16_byte_aligned(shape):
    # C two bytes past a 16-byte boundary (bf16 out, ldc a multiple of 8):
    # the 16-byte LDS-staged stores are off, the per-element epilogue runs;
    # nothing is written before C or outside the M x N block.
    M, N, K = shape
    announce("C base + 2 bytes", M, N, K)
    p = H.problem(M, N, K, synth.BF16, "K", "MN", "int", (121, 122))
    A, B = H.to_device(p.A), H.to_device(p.B)
    ldc = N + 8
    buf = torch.full((M * ldc + 16,), int(H.CANARY_U16), dtype=torch.int16, device="cuda")
    st = lsm.gemm_run(H.handle(), A, B, buf.data_ptr() + 2, M, N, K, p.lda, p.ldb, ldc,
                      H.LAYOUT["K"], H.LAYOUT["MN"], lsm.GEMM_BF16_BF16, torch.cuda.current_stream())
    assert st == lsm.GEMM_OK
    torch.cuda.synchronize()
    host = buf.cpu().numpy().view(np.uint16)
    assert host[0] == H.CANARY_U16
    C = host[1:1 + M * ldc].reshape(M, ldc)
    H.assert_canary(C, M, N, lsm.GEMM_BF16_BF16)
    rng = np.random.default_rng(2)
    for r0, r1 in ((0, 2), (M - 2, M)):
        H.assert_exact(C[r0:r1, :N], H.oracle_rows(p, r0, r1), lsm.GEMM_BF16_BF16, f"rows {r0}")
    rows, cols = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
    H.assert_exact(C[rows, cols], H.oracle_entries(p, rows, cols), lsm.GEMM_BF16_BF16, "entries")


def sample_check(p, C, gdtype, exact, rows_sel, n_entries=4000, seed=0):
    rng = np.random.default_rng(seed)
    for r0, r1 in rows_sel:
        ref = H.oracle_rows(p, r0, r1)
        if exact:
            H.assert_exact(C[r0:r1, :p.N], ref, gdtype, f"rows {r0}:{r1}")
        else:
            H.assert_close(C[r0:r1, :p.N], ref, p.K, gdtype, f"rows {r0}:{r1}")
    rows, cols = rng.integers(0, p.M, n_entries), rng.integers(0, p.N, n_entries)
    ref = H.oracle_entries(p, rows, cols)
    if exact:
        H.assert_exact(C[rows, cols], ref, gdtype, "entries")
    else:
        H.assert_close(C[rows, cols], ref, p.K, gdtype, "entries")


def every_tile_check(p, C, gdtype, exact, seed=0):
    """A full row in every 256-row tile row and a full column in every
    256-column tile column of C against the oracle: every 256 x 256 tile of
    the launch has a checked row and a checked column."""
    rows, cols = H.every_tile_rows_cols(p.M, p.N, 256, seed)
    ref_r = H.oracle_row_set(p, rows)
    ref_c = H.oracle_col_set(p, cols)
    got_r = C[rows, :p.N]
    got_c = np.ascontiguousarray(C[:p.M, cols].T)
    if exact:
        H.assert_exact(got_r, ref_r, gdtype, "tile rows")
        H.assert_exact(got_c, ref_c, gdtype, "tile columns")
    else:
        H.assert_close(got_r, ref_r, p.K, gdtype, "tile rows")
        H.assert_close(got_c, ref_c, p.K, gdtype, "tile columns")


@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_config_4096_all_layouts_bf16_out(la, lb):
    w = synth.WORKLOADS["bf16_4096_all_bf16"]
    announce(4096, la, lb)
    p = H.problem(4096, 4096, 4096, synth.BF16, la, lb, w["dist"], w["seeds"])
    C = H.run_gpu(p, lsm.GEMM_BF16_BF16)
    every_tile_check(p, C, lsm.GEMM_BF16_BF16, False, seed=3)
    sample_check(p, C, lsm.GEMM_BF16_BF16, False, [], 3000)


@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_config_4096_integer_exact(la, lb):
    announce(4096, "int", la, lb)
    p = H.problem(4096, 4096, 4096, synth.BF16, la, lb, "int", (3001, 3002))
    C = H.run_gpu(p, lsm.GEMM_BF16_BF16)
    every_tile_check(p, C, lsm.GEMM_BF16_BF16, True, seed=4)
    sample_check(p, C, lsm.GEMM_BF16_BF16, True, [], 3000)


def test_config_8192_nn_f32():
    w = synth.WORKLOADS["bf16_8192_nn_f32"]
    announce(8192, "normal")
    p = H.problem(8192, 8192, 8192, synth.BF16, "K", "MN", w["dist"], w["seeds"])
    C = H.run_gpu(p, lsm.GEMM_BF16_F32)
    every_tile_check(p, C, lsm.GEMM_BF16_F32, False, seed=5)
    sample_check(p, C, lsm.GEMM_BF16_F32, False, [], 2000)


def test_config_8192_integer_exact():
    announce(8192, "int")
    p = H.problem(8192, 8192, 8192, synth.BF16, "K", "MN", "int", (4001, 4002))
    C = H.run_gpu(p, lsm.GEMM_BF16_F32)
    every_tile_check(p, C, lsm.GEMM_BF16_F32, True, seed=6)
    sample_check(p, C, lsm.GEMM_BF16_F32, True, [], 2000)


# M <= 32 with whole 16-byte chunks along every contiguous extent: the
# streaming skinny kernel (deep direct-to-LDS ring, K split over the waves,
# partial sums reduced in LDS).  Partial last K stage, K shorter than the
# ring, ragged N, odd M where A is K-contiguous.
SKINNY_DMA = [(8, 136, 264), (32, 1000, 1032), (24, 4160, 520), (16, 64, 8), (32, 8, 128),
              (8, 200, 3208)]
SKINNY_DMA_KA = [(1, 520, 1000), (31, 264, 136), (17, 72, 2056)]


@pytest.mark.parametrize("shape", SKINNY_DMA)
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_skinny_stream_integer_exact(shape, la, lb):
    M, N, K = shape
    check_full(M, N, K, la, lb, lsm.GEMM_BF16_F32, "int", (91, 92), ldc_pad=3, extra_rows=2)


@pytest.mark.parametrize("shape", SKINNY_DMA_KA)
@pytest.mark.parametrize("lb", ["MN", "K"])
def test_skinny_stream_odd_m_integer_exact(shape, lb):
    M, N, K = shape
    check_full(M, N, K, "K", lb, lsm.GEMM_BF16_F32, "int", (93, 94), ldc_pad=1, extra_rows=1)


@pytest.mark.parametrize("gdtype", ALL_DTYPES)
@pytest.mark.parametrize("la,lb", [("K", "MN"), ("MN", "K")])
def test_skinny_stream_real_all_dtypes(gdtype, la, lb):
    check_full(24, 1160, 1544, la, lb, gdtype, "normal", (95, 96), ldc_pad=5, extra_rows=1)


def test_config_skinny_bf16_out():
    w = synth.WORKLOADS["bf16_skinny_32x16384x8192_nn_bf16"]
    announce("skinny")
    p = H.problem(32, 16384, 8192, synth.BF16, "K", "MN", w["dist"], w["seeds"])
    C = H.run_gpu(p, lsm.GEMM_BF16_BF16)
    ref = H.oracle_full(p)
    H.assert_close(C, ref, 8192, lsm.GEMM_BF16_BF16, "skinny")


def test_config_skinny_integer_exact():
    announce("skinny int")
    p = H.problem(32, 16384, 8192, synth.BF16, "K", "MN", "int", (5001, 5002))
    C = H.run_gpu(p, lsm.GEMM_BF16_BF16)
    H.assert_exact(C, H.oracle_full(p), lsm.GEMM_BF16_BF16, "skinny int")


# ------------------------------------------------------------------ ABI behaviour on the GPU

@pytest.mark.parametrize("big", ["A", "B"])
def test_operand_footprint_beyond_2gib(big):
    # An operand whose footprint passes 2^31 bytes (72 rows of a 2^24 + 72
    # element leading dimension, 2.4 GB) is beyond the 32-bit buffer offsets
    # of the direct-to-LDS kernels: the register-staged kernel with 64-bit
    # addressing takes it, bit-exact against the oracle.
    M, N, K = 72, 200, 72
    wide = (1 << 24) + 72 - K if big == "A" else (1 << 24) + 72 - N
    announce("footprint > 2 GiB", big, M, N, K)
    p = synth.make_problem(M, N, K, synth.BF16, "K", "MN", "int", 31, 32,
                           pad_a=wide if big == "A" else 0, pad_b=wide if big == "B" else 0)
    fp = (((M - 1) * p.lda + K) if big == "A" else ((K - 1) * p.ldb + N)) * 2
    assert fp > (1 << 31)
    C = H.run_gpu(p, lsm.GEMM_BF16_F32, ldc=N + 8, extra_rows=1)
    H.assert_canary(C, M, N, lsm.GEMM_BF16_F32)
    H.assert_exact(C[:M, :N], H.oracle_full(p), lsm.GEMM_BF16_F32, f"footprint {big}")


def test_error_paths_leave_c_untouched():
    announce("errors")
    h = H.handle()
    A = torch.zeros(4096, dtype=torch.int16, device="cuda")
    B = torch.zeros(4096, dtype=torch.int16, device="cuda")
    C = torch.full((4096,), 7.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    ok = lambda *a: lsm.gemm_run(h, *a, s)
    # misaligned A pointer (2 bytes off) -> unsupported
    assert ok(A.data_ptr() + 2, B, C, 16, 16, 16, 16, 16, 16, 0, 1, 0) == lsm.GEMM_ERR_UNSUPPORTED
    # lda not a multiple of 8 -> unsupported
    assert ok(A, B, C, 16, 16, 12, 12, 16, 16, 0, 1, 0) == lsm.GEMM_ERR_UNSUPPORTED
    # C overlapping A -> invalid
    assert ok(A, B, A, 16, 16, 16, 16, 16, 16, 0, 1, 1) == lsm.GEMM_ERR_INVALID_ARG
    # bad enums / sizes -> invalid
    assert ok(A, B, C, 16, 16, 16, 16, 16, 16, 2, 1, 0) == lsm.GEMM_ERR_INVALID_ARG
    assert ok(A, B, C, 16, 16, 16, 16, 16, 16, 0, 1, 9) == lsm.GEMM_ERR_INVALID_ARG
    assert ok(A, B, C, -1, 16, 16, 16, 16, 16, 0, 1, 0) == lsm.GEMM_ERR_INVALID_ARG
    assert ok(A, B, C, 16, 16, 16, 8, 16, 16, 0, 1, 0) == lsm.GEMM_ERR_INVALID_ARG
    # M == 0 and N == 0 are no-ops
    assert ok(A, B, C, 0, 16, 16, 16, 16, 16, 0, 1, 0) == lsm.GEMM_OK
    assert ok(A, B, C, 16, 0, 16, 16, 16, 16, 0, 1, 0) == lsm.GEMM_OK
    torch.cuda.synchronize()
    assert bool(torch.all(C == 7.0))


def test_runs_on_a_side_stream():
    announce("side stream")
    p = H.problem(512, 384, 320, synth.BF16, "K", "MN", "int", (81, 82))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = H.run_gpu(p, lsm.GEMM_BF16_F32, stream=s)
    H.assert_exact(C, H.oracle_full(p), lsm.GEMM_BF16_F32, "side stream")
