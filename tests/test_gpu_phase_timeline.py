"""The measurement builds `timeline` and `timeline1` (ping-pong kernel with
per-wave phase cycle counts; the second on one loader group): with a count
buffer installed they still compute the library's product bit for bit, every
wave of every workgroup writes its counts, and the per-phase sums fit inside
the K loop they were taken in.  With no buffer installed they write nothing
(the A/B parity test runs them that way)."""
import ctypes

import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
from lds_staged_matrix_amd import build as hip_build
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["timeline", "timeline1"])
@pytest.mark.parametrize("la,lb", [("K", "MN"), ("MN", "MN")])
def test_timeline_build_counts_and_stays_exact(name, la, lb):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M, N, K = 4096, 4096, 520          # 256 ping-pong workgroups, 9 K tiles, the last partial
    print("CASE timeline", name, la, lb, M, N, K, flush=True)
    p = H.problem(M, N, K, synth.BF16, la, lb, "int", (301, 302))
    ref = H.run_gpu(p, lsm.GEMM_BF16_F32)
    lib = lsm.ablation_library(name)
    raw = ctypes.CDLL(hip_build.variant_path(name))
    raw.lsm_pp_timeline_set.argtypes = [ctypes.c_void_p]
    raw.lsm_pp_timeline_set.restype = ctypes.c_int
    wgs = (M // 256) * (N // 256)
    buf = torch.zeros(wgs * 64, dtype=torch.int64, device="cuda")
    h = lib.gemm_create()
    assert raw.lsm_pp_timeline_set(buf.data_ptr()) == 0
    try:
        got = H.run_gpu(p, lsm.GEMM_BF16_F32, lib=(lib, h))
    finally:
        assert raw.lsm_pp_timeline_set(None) == 0
        lib.gemm_destroy(h)
    assert np.array_equal(got, ref), f"{name} differs from the library"
    t = buf.cpu().numpy().reshape(wgs, 8, 8)
    phases, prologue, loop, epilogue = t[:, :, :5], t[:, :, 5], t[:, :, 6], t[:, :, 7]
    assert (loop > 0).all() and (prologue > 0).all() and (epilogue > 0).all(), "a wave wrote no counts"
    assert (phases >= 0).all()
    assert (phases[:, :, 2] > 0).all(), "MFMA issue counted on every wave"
    assert (phases.sum(axis=2) <= loop).all(), "phases outside the K loop"
    # group 1 waits for no loads of its own at the end of its compute phase
    assert (phases[:, 4:, 3] == 0).all()
