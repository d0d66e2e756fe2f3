"""The A/B builds (one design choice changed each: no LDS swizzle, scalar
16-bit reads instead of ds_read_b64_tr_b16, a 2-stage ring for M <= 32,
tiles in hardware workgroup order instead of the per-XCD order, one LDS
stage instead of two in the direct-to-LDS kernel, the 64 x 64 tile without
its four-stage pipeline, 32 x 32 MFMAs in the ping-pong kernel, the
ping-pong kernel staging C per wave instead of per workgroup, the ping-pong
kernel with one loader group instead of loads split between its groups)
compute the same products: bit-identical to the library on integer-valued
inputs, whose result is unique.  Their speed and counters are what the
benchmark compares; this checks that they are the same computation."""
import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

VARIANTS = ["noswizzle", "scalar_tr", "ring2", "noxcd", "stage1", "small2", "mfma32", "waveepi", "oneloader", "timeline", "timeline1"]
# one shape per kernel: ping-pong (>= 256 tiles of 256), 128 x 128 tile
# (>= 256 tiles of 128), 64 x 64 tile with two and with four LDS stages (its
# operand panels beyond one XCD's L2), split-K ring (M <= 32)
SHAPES = [(4096, 4096, 136), (2048, 2056, 200), (520, 264, 1000), (500, 300, 6152),
          (32, 1000, 1032)]
LAYOUTS = [("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")]


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    out = {}
    for v in VARIANTS:
        lib = lsm.ablation_library(v)
        out[v] = (lib, lib.gemm_create())
    yield out
    for lib, h in out.values():
        lib.gemm_destroy(h)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_ablation_builds_match_the_library(libs, shape, la, lb):
    M, N, K = shape
    print("CASE ablation", M, N, K, la, lb, flush=True)
    p = H.problem(M, N, K, synth.BF16, la, lb, "int", (101, 102))
    ref = H.run_gpu(p, lsm.GEMM_BF16_F32)
    rows = sorted({0, M // 2, M - 1})
    H.assert_exact(ref[rows, :], H.oracle_entries(p, np.repeat(rows, N), np.tile(np.arange(N), len(rows))).reshape(len(rows), N),
                   lsm.GEMM_BF16_F32, "library rows")
    A, B = H.to_device(p.A), H.to_device(p.B)
    for v, (lib, h) in libs.items():
        C = torch.full((M * N,), float(H.CANARY_F32), dtype=torch.float32, device="cuda")
        st = lib.gemm_run(h, A, B, C, M, N, K, p.lda, p.ldb, N, H.LAYOUT[la], H.LAYOUT[lb],
                          lsm.GEMM_BF16_F32, torch.cuda.current_stream())
        assert st == lsm.GEMM_OK, (v, st)
        torch.cuda.synchronize()
        got = C.cpu().numpy().reshape(M, N)
        assert np.array_equal(got, ref), f"{v} differs from the library"
