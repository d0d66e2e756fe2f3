"""Edge chunks of the direct-to-LDS kernels read as zero, not as whatever
follows the operand in memory.

The direct-to-LDS loads reach their edges through the buffer range check:
each operand's buffer resource holds its exact footprint
((rows - 1) * ld + row length, in bytes), and the K advance and the load round
ride in the scalar offset, so the rows past K of an MN-contiguous operand in
the last, partial K tile and the rows past M or N in later load rounds are
loads whose vector offset is in range and whose vector plus scalar offset is
not.  The hardware probe test pins that such loads return zeros; this test
checks the kernels end to end.  Every operand here sits at the very end of its
allocation's live bytes, followed at once by a guard of NaN bytes inside the
same allocation (all-ones bytes: NaN as bf16, fp16 and E4M3).  A kernel that
read past the footprint would meet the guard and put NaN into the result.
The guard spans a whole tile of rows past the footprint, so no access can
leave the allocation.  Every direct-to-LDS kernel class runs with ragged M and
N and a partial last K tile, in all four layouts, on integer inputs (a
unique, bit-exact result).
"""
import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
import synth
import gpu_harness as H
from test_gpu_every_kernel import shape_class

pytestmark = pytest.mark.gpu

ALL_LAYOUTS = [("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")]
# (class, M, N, K): K one chunk past a whole number of K tiles (BK 64 for the
# 16-bit tiles, 128 for the split-K ring's stages; twice that for E4M3)
CASES16 = [
    ("pingpong", 4104, 4088, 72),
    ("dma128", 2056, 2048, 72),
    ("dma64", 520, 264, 136),
    ("dma64x4", 512, 520, 4104),
    ("ring", 32, 1000, 1032),
]
CASES8 = [
    ("pingpong", 4112, 4096, 144),
    ("dma128", 2064, 2048, 144),
    ("dma64", 528, 272, 272),
    ("ring", 32, 1024, 1040),
]


def guarded(bits, footprint_elems, guard_bytes):
    """Device copy of the first `footprint_elems` elements of an operand,
    followed in the same allocation by `guard_bytes` bytes of 0xFF."""
    raw = np.ascontiguousarray(bits).reshape(-1)[:footprint_elems].view(np.uint8)
    host = np.concatenate([raw, np.full(guard_bytes, 0xFF, np.uint8)])
    return torch.from_numpy(host).to("cuda")


def run_guarded(p, gd):
    es = 1 if p.dtype == synth.E4M3 else 2
    a_outer, a_inner = (p.M, p.K) if p.layoutA == "K" else (p.K, p.M)
    b_outer, b_inner = (p.K, p.N) if p.layoutB == "MN" else (p.N, p.K)
    a_fp = (a_outer - 1) * p.lda + a_inner
    b_fp = (b_outer - 1) * p.ldb + b_inner
    # a tile of rows (256) past the footprint, and then some
    A = guarded(p.A, a_fp, 256 * p.lda * es + (64 << 10))
    B = guarded(p.B, b_fp, 256 * p.ldb * es + (64 << 10))
    out_f32 = H.OUT_OF[gd] == "f32"
    C = torch.empty(p.M * p.N, dtype=torch.float32 if out_f32 else torch.int16, device="cuda")
    st = lsm.gemm_run(H.handle(), A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.N,
                      H.LAYOUT[p.layoutA], H.LAYOUT[p.layoutB], gd, torch.cuda.current_stream())
    assert st == lsm.GEMM_OK
    torch.cuda.synchronize()
    host = C.cpu().numpy()
    return (host if out_f32 else host.view(np.uint16)).reshape(p.M, p.N)


def check(cls, M, N, K, la, lb, gd, seed):
    es = 1 if H.IN_OF[gd] == synth.E4M3 else 2
    assert shape_class(M, N, K, la, lb, es) == cls
    print(f"CASE guard-region {cls} {M}x{N}x{K} {la}{lb} dtype {gd}", flush=True)
    p = H.problem(M, N, K, H.IN_OF[gd], la, lb, "int", (seed, seed + 1))
    C = run_guarded(p, gd)
    # every row of the last tile row and column, and a sample elsewhere
    rows = sorted(set(range(max(0, M - 40), M)) | {0, M // 2})
    want = H.oracle_entries(p, np.repeat(rows, N), np.tile(np.arange(N), len(rows)))
    H.assert_exact(C[rows, :], want.reshape(len(rows), N), gd, f"{cls} {la}{lb} rows")
    cols = np.arange(max(0, N - 40), N)
    r = np.repeat(np.arange(M), len(cols))
    c = np.tile(cols, M)
    H.assert_exact(C[r, c], H.oracle_entries(p, r, c), gd, f"{cls} {la}{lb} last columns")


@pytest.mark.parametrize("case", CASES16, ids=lambda c: c[0])
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
@pytest.mark.parametrize("gd", [lsm.GEMM_BF16_F32, lsm.GEMM_F16_F16])
def test_guard_after_each_operand_16bit(case, la, lb, gd):
    check(*case, la, lb, gd, 1200 + 10 * gd)


@pytest.mark.parametrize("case", CASES8, ids=lambda c: c[0])
@pytest.mark.parametrize("la,lb", ALL_LAYOUTS)
def test_guard_after_each_operand_8bit(case, la, lb):
    check(*case, la, lb, lsm.GEMM_E4M3_F32, 1300)
