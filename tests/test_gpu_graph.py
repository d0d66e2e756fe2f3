"""gemm_run under HIP graph capture: the call only enqueues kernels on the
given stream (no allocation, no synchronisation, no memset), so it can be
captured.  Every replay, with eager work and synchronisations between the
replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import lds_staged_matrix_amd as lsm
import synth
import gpu_harness as H

pytestmark = pytest.mark.gpu

# one shape per kernel: ping-pong, 128 x 128, 64 x 64, split-K ring, register-staged
SHAPES = [((4096, 4096, 136), "K", "MN"), ((2048, 2056, 200), "K", "K"),
          ((520, 264, 1000), "MN", "MN"), ((32, 1000, 1032), "K", "MN"),
          ((100, 96, 17), "K", "MN")]


@pytest.mark.parametrize("shape,la,lb", SHAPES)
def test_graph_replays_match_eager(shape, la, lb):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M, N, K = shape
    print("CASE graph", M, N, K, la, lb, flush=True)
    p = H.problem(M, N, K, synth.BF16, la, lb, "int", (131, 132))
    A, B = H.to_device(p.A), H.to_device(p.B)
    h = H.handle()
    gd = lsm.GEMM_BF16_F32
    eager = torch.full((M * N,), float("nan"), dtype=torch.float32, device="cuda")
    assert lsm.gemm_run(h, A, B, eager, M, N, K, p.lda, p.ldb, N, H.LAYOUT[la], H.LAYOUT[lb], gd,
                        torch.cuda.current_stream()) == lsm.GEMM_OK
    torch.cuda.synchronize()
    rows = sorted({0, M // 2, M - 1})
    H.assert_exact(eager.view(M, N)[rows].cpu().numpy(),
                   H.oracle_entries(p, np.repeat(rows, N), np.tile(np.arange(N), len(rows)))
                   .reshape(len(rows), N), gd, "eager rows")

    C = torch.empty(M * N, dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            st = lsm.gemm_run(h, A, B, C, M, N, K, p.lda, p.ldb, N, H.LAYOUT[la], H.LAYOUT[lb],
                              gd, torch.cuda.current_stream())
    assert st == lsm.GEMM_OK
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        C.fill_(float("nan"))                # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), eager.view(torch.int32)), f"replay {rep}"
