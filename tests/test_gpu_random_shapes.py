"""Seeded random sweep: shapes, layouts, element types, leading-dimension
padding and ldc, each checked bit for bit against the oracle on integer
inputs (whose result is unique).  Sizes stay small enough for the oracle to
compute every entry; they straddle every kernel class (M <= 32, 64/128/256
tiles, register-staged shapes with odd contiguous extents) and their edges."""
import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

LAYOUTS = [("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")]
DTYPES_16 = [lsm.GEMM_BF16_F32, lsm.GEMM_BF16_BF16, lsm.GEMM_F16_F16, lsm.GEMM_F16_F32]
DTYPES_8 = [lsm.GEMM_E4M3_F32, lsm.GEMM_E4M3_BF16]


def cases(n=48, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fp8 = i % 6 == 5
        kind = rng.integers(0, 4)
        if kind == 0:
            M = int(rng.integers(1, 33))                               # split-K ring
        elif kind == 1:
            M = int(rng.integers(33, 400))                             # 64 / 128 tiles
        else:
            M = int(rng.integers(400, 1300))
        N = int(rng.integers(1, 1300))
        K = int(rng.integers(1, 700))
        la, lb = LAYOUTS[int(rng.integers(0, 4))]
        if fp8:                                                        # 16-element extents
            K = max(16, K // 16 * 16)
            if la == "MN":
                M = max(16, M // 16 * 16)
            if lb == "MN":
                N = max(16, N // 16 * 16)
            gd = DTYPES_8[int(rng.integers(0, 2))]
        else:
            gd = DTYPES_16[int(rng.integers(0, 4))]
        out.append((i, M, N, K, la, lb, gd, int(rng.integers(0, 3)), int(rng.integers(0, 9))))
    return out


@pytest.mark.parametrize("case", cases(), ids=lambda c: f"c{c[0]}")
def test_random_shape_integer_exact(case):
    i, M, N, K, la, lb, gd, pad, ldc_pad = case
    print("CASE random", i, M, N, K, la, lb, gd, pad, ldc_pad, flush=True)
    p = H.problem(M, N, K, H.IN_OF[gd], la, lb, "int", (500 + i, 600 + i), extra_pad=pad)
    C = H.run_gpu(p, gd, ldc=N + ldc_pad, extra_rows=1)
    H.assert_canary(C, M, N, gd)
    H.assert_exact(C[:M, :N], H.oracle_full(p), gd, f"case {i}")
