"""One handle used from several host threads and streams at once.

The header promises that a handle is immutable after creation, so gemm_run may
be called concurrently from several threads on several streams.  Four threads,
each with its own stream, launch different shape classes (ping-pong, 128 and
64 direct-to-LDS tiles, split-K ring) on shared read-only operands, three
times each; every output is compared bit for bit with the oracle (integer
inputs: the result is unique).
"""
import threading

import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

CASES = [  # (M, N, K, layoutA, layoutB, dtype)
    (4096, 4096, 128, "K", "MN", lsm.GEMM_BF16_F32),     # ping-pong, 256 tiles
    (2048, 2048, 200, "K", "K", lsm.GEMM_BF16_BF16),     # 128 x 128 tiles
    (520, 264, 136, "MN", "MN", lsm.GEMM_F16_F16),       # 64 x 64 tiles
    (32, 4096, 512, "K", "MN", lsm.GEMM_BF16_BF16),      # split-K ring, M <= 32
]
REPEATS = 3


def test_one_handle_many_threads_and_streams():
    print("CASE concurrency: 4 threads x 4 streams, one handle", flush=True)
    h = H.handle()
    probs, expect, devs = [], [], []
    for i, (M, N, K, la, lb, gd) in enumerate(CASES):
        p = H.problem(M, N, K, H.IN_OF[gd], la, lb, "int", (900 + 2 * i, 901 + 2 * i))
        probs.append(p)
        expect.append(H.oracle_full(p))
        devs.append((H.to_device(p.A), H.to_device(p.B)))
    torch.cuda.synchronize()
    outs = [[None] * REPEATS for _ in CASES]
    errors = []
    start = threading.Barrier(len(CASES))

    def worker(i):
        try:
            M, N, K, la, lb, gd = CASES[i]
            p = probs[i]
            A, B = devs[i]
            s = torch.cuda.Stream()
            f32 = H.OUT_OF[gd] == "f32"
            with torch.cuda.stream(s):
                Cs = [torch.empty(M * N, dtype=torch.float32 if f32 else torch.int16, device="cuda")
                      for _ in range(REPEATS)]
            s.synchronize()
            start.wait()
            for r in range(REPEATS):
                st = lsm.gemm_run(h, A, B, Cs[r], M, N, K, p.lda, p.ldb, N, H.LAYOUT[la],
                                  H.LAYOUT[lb], gd, s)
                if st != lsm.GEMM_OK:
                    raise lsm.GemmError(st, "gemm_run")
            s.synchronize()
            for r in range(REPEATS):
                outs[i][r] = Cs[r].cpu().numpy().reshape(M, N)
        except Exception as e:  # reported by the main thread
            errors.append((i, e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    for i, (M, N, K, la, lb, gd) in enumerate(CASES):
        for r in range(REPEATS):
            got = outs[i][r]
            if H.OUT_OF[gd] != "f32":
                got = got.view(np.uint16)
            H.assert_exact(got, expect[i], gd, f"thread {i} launch {r} {M}x{N}x{K} {la}{lb}")
