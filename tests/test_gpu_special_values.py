"""IEEE special values and subnormals through the kernels, against the oracle.

The oracle decodes every input bit pattern exactly (its decoders are pinned on
all 65536 bf16/fp16 and all 256 E4M3 patterns) and sums in fp64, so NaN, Inf,
Inf*0 and subnormal operands follow IEEE arithmetic there.  The GPU result
must put NaN and +-Inf in the same places and, where every product and partial
sum is exact in fp32 (the cases below are built that way), match the finite
values bit for bit: matrix-core inputs and fp32 results that are subnormal are
kept, not flushed.
"""
import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
import oracle
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

ONE = {synth.BF16: 0x3F80, synth.F16: 0x3C00, synth.E4M3: 0x38}
NAN = {synth.BF16: 0x7FC0, synth.F16: 0x7E00, synth.E4M3: 0x7F}
PINF = {synth.BF16: 0x7F80, synth.F16: 0x7C00}
STORE = {synth.BF16: np.uint16, synth.F16: np.uint16, synth.E4M3: np.uint8}


def run_nn(A, B, M, N, K, gd):
    """C = A*B with A K-contiguous (lda = K) and B N-contiguous (ldb = N);
    returns the output decoded to float64."""
    dA, dB = H.to_device(A.reshape(-1)), H.to_device(B.reshape(-1))
    f32 = H.OUT_OF[gd] == "f32"
    C = torch.zeros(M * N, dtype=torch.float32 if f32 else torch.int16, device="cuda")
    st = lsm.gemm_run(H.handle(), dA, dB, C, M, N, K, K, N, N, lsm.GEMM_K_CONTIG,
                      lsm.GEMM_MN_CONTIG, gd, torch.cuda.current_stream())
    assert st == lsm.GEMM_OK, lsm.gemm_status_str(st)
    torch.cuda.synchronize()
    got = C.cpu().numpy().reshape(M, N)
    return H.gpu_values(got if f32 else got.view(np.uint16), gd)


def ref_nn(A, B, M, N, K, dtype):
    return oracle.gemm(A.reshape(-1), B.reshape(-1), M, N, K, K, N, oracle.K_CONTIG,
                       oracle.MN_CONTIG, H.ODTYPE[dtype])


def assert_same_specials(got, ref, what, gd):
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN positions differ"
    assert np.array_equal(np.isposinf(got), np.isposinf(ref)), f"{what}: +Inf positions differ"
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -Inf positions differ"
    fin = np.isfinite(ref)
    if H.OUT_OF[gd] == "f32":
        assert np.array_equal(got[fin], ref[fin]), f"{what}: finite values differ"
    else:
        want = oracle.decode(oracle.encode(ref[fin], oracle.BF16 if H.OUT_OF[gd] == "bf16"
                                           else oracle.F16), oracle.BF16 if H.OUT_OF[gd] == "bf16"
                             else oracle.F16)
        assert np.array_equal(got[fin], want), f"{what}: finite values differ"


SHAPES = [(64, 64, 64), (4096, 4096, 64)]   # the 64 x 64 kernel and the ping-pong kernel


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("gd", [lsm.GEMM_BF16_F32, lsm.GEMM_BF16_BF16, lsm.GEMM_F16_F16,
                                lsm.GEMM_E4M3_F32])
def test_nan_inf_propagate(shape, gd):
    M, N, K = shape
    dt = H.IN_OF[gd]
    print(f"CASE special values {M}x{N}x{K} dtype {gd}", flush=True)
    A = np.full((M, K), ONE[dt], STORE[dt])
    B = np.full((K, N), ONE[dt], STORE[dt])
    A[3, 5] = NAN[dt]                          # row 3 of C: NaN
    if dt != synth.E4M3:                       # E4M3 has no infinities
        B[7, 9] = PINF[dt]                     # column 9 of C: +Inf (row 3 stays NaN)
        A[10, 0] = 0                           # 0 * +Inf at (10, 20): NaN
        B[0, 20] = PINF[dt]
        B[1, 30] = PINF[dt] | 0x8000           # column 30: -Inf
    got, ref = run_nn(A, B, M, N, K, gd), ref_nn(A, B, M, N, K, dt)
    assert np.isnan(ref[3]).all() and (dt == synth.E4M3 or np.isnan(ref[10, 20]))
    assert_same_specials(got, ref, f"{M}x{N}x{K} {gd}", gd=gd)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt,sub,scale", [
    (synth.BF16, range(1, 128), 0x7180),       # m * 2^-133 times 2^100
    (synth.F16, range(1, 1024), 0x6400),       # m * 2^-24 times 2^10
    (synth.E4M3, range(1, 8), 0x68),           # m * 2^-9 times 2^6
])
def test_subnormal_inputs_are_kept(shape, dt, sub, scale):
    M, N, K = shape
    gd = {synth.BF16: lsm.GEMM_BF16_F32, synth.F16: lsm.GEMM_F16_F32,
          synth.E4M3: lsm.GEMM_E4M3_F32}[dt]
    print(f"CASE subnormal inputs {M}x{N}x{K} {dt}", flush=True)
    pats = np.array(list(sub), dtype=STORE[dt])
    A = np.zeros((M, K), STORE[dt])
    B = np.zeros((K, N), STORE[dt])
    A[:, 0] = pats[np.arange(M) % pats.size]   # one subnormal per row, in column k = 0
    B[0, :] = scale                            # products below 1, exact in fp32
    got, ref = run_nn(A, B, M, N, K, gd), ref_nn(A, B, M, N, K, dt)
    assert (ref[:, 1] != 0).all() and (ref[:, 1] < 1).all()   # subnormal-born, nonzero values
    assert_same_specials(got, ref, f"subnormal {dt}", gd=gd)


def test_subnormal_fp32_result_is_kept():
    """bf16 2^-100 times 2^-40 = 2^-140: an fp32 subnormal, written as such."""
    print("CASE fp32 subnormal result", flush=True)
    M = N = K = 64
    A = np.zeros((M, K), np.uint16)
    B = np.zeros((K, N), np.uint16)
    A[:, 0] = 0x0D80                           # 2^-100
    B[0, :] = 0x2B80                           # 2^-40
    got = run_nn(A, B, M, N, K, lsm.GEMM_BF16_F32)
    ref = ref_nn(A, B, M, N, K, synth.BF16)
    assert ref[0, 0] == 2.0 ** -140
    assert np.array_equal(got, ref)
