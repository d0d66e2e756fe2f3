"""Shared helpers of the GPU tests: move synthetic problems to the device, call
the C ABI through the Python binding, and compare with the oracle.

The comparison rules:
  * integer-valued inputs (entries in {-2..2}): every product and partial sum
    is an integer below 2^24, so fp32 accumulation is exact and the result is
    unique; the GPU output must equal the oracle's exact sum rounded once to
    the output type (round to nearest even), bit for bit;
  * real-valued inputs: fp32 output within |c - ref| <= 1e-5*K, bf16 output
    within 2^-8*|ref| + 1e-5*K, fp16 output within 2^-11*|ref| + 1e-5*K
    (the fp16 rule is the bf16 rule with fp16's half-ulp).
"""
import numpy as np
import torch

import lds_staged_matrix_amd as lsm
import oracle
import synth

OUT_OF = {lsm.GEMM_BF16_F32: "f32", lsm.GEMM_BF16_BF16: "bf16", lsm.GEMM_F16_F16: "f16",
          lsm.GEMM_F16_F32: "f32", lsm.GEMM_E4M3_F32: "f32", lsm.GEMM_E4M3_BF16: "bf16"}
IN_OF = {lsm.GEMM_BF16_F32: synth.BF16, lsm.GEMM_BF16_BF16: synth.BF16,
         lsm.GEMM_F16_F16: synth.F16, lsm.GEMM_F16_F32: synth.F16,
         lsm.GEMM_E4M3_F32: synth.E4M3, lsm.GEMM_E4M3_BF16: synth.E4M3}
LAYOUT = {"K": lsm.GEMM_K_CONTIG, "MN": lsm.GEMM_MN_CONTIG}
OLAYOUT = {"K": oracle.K_CONTIG, "MN": oracle.MN_CONTIG}
ODTYPE = {synth.BF16: oracle.BF16, synth.F16: oracle.F16, synth.E4M3: oracle.E4M3}
CANARY_F32 = np.float32(-12345.5)
CANARY_U16 = np.uint16(0x5A5A)

_handle = None


def handle():
    global _handle
    if _handle is None:
        _handle = lsm.gemm_create()
    return _handle


def ld_pad(extent, extra=0, dtype=synth.BF16):
    """Padding that makes the leading dimension a multiple of 16 bytes
    (8 bf16/fp16 or 16 e4m3 elements)."""
    q = 16 if dtype == synth.E4M3 else 8
    return (-max(extent, 1)) % q + q * extra


def problem(M, N, K, dtype, la, lb, dist, seeds=(1, 2), scale=1.0, extra_pad=0):
    inner_a = K if la == "K" else M
    inner_b = N if lb == "MN" else K
    return synth.make_problem(M, N, K, dtype, la, lb, dist, seeds[0], seeds[1], scale,
                              pad_a=ld_pad(inner_a, extra_pad, dtype),
                              pad_b=ld_pad(inner_b, extra_pad, dtype))


def to_device(bits):
    raw = np.ascontiguousarray(bits)
    b = raw.view(np.int8) if raw.dtype == np.uint8 else raw.view(np.int16)
    if b.size == 0:
        return torch.empty(16, dtype=torch.int16, device="cuda")
    return torch.from_numpy(b).to("cuda")


def run_gpu(p, gdtype, ldc=None, extra_rows=0, stream=None, lib=None):
    """C = A*B on the GPU.  Returns (C as numpy: float32 values or uint16 bits,
    shape (M + extra_rows, ldc)), with canary values outside the M x N block.
    `lib` = (Library, handle) runs an A/B build instead of the library."""
    M, N, K = p.M, p.N, p.K
    ldc = N if ldc is None else ldc
    rows = M + extra_rows
    out = OUT_OF[gdtype]
    A, B = to_device(p.A), to_device(p.B)
    if out == "f32":
        C = torch.full((max(rows * ldc, 1),), float(CANARY_F32), dtype=torch.float32, device="cuda")
    else:
        C = torch.full((max(rows * ldc, 1),), int(CANARY_U16), dtype=torch.int16, device="cuda")
    s = torch.cuda.current_stream() if stream is None else stream
    run, h = (lsm.gemm_run, handle()) if lib is None else (lib[0].gemm_run, lib[1])
    st = run(h, A, B, C, M, N, K, p.lda, p.ldb, ldc, LAYOUT[p.layoutA], LAYOUT[p.layoutB],
             gdtype, s)
    if st != lsm.GEMM_OK:
        raise lsm.GemmError(st, "gemm_run")
    torch.cuda.synchronize()
    host = C.cpu().numpy()
    if out != "f32":
        host = host.view(np.uint16)
    return host[: rows * ldc].reshape(rows, ldc) if rows * ldc else host[:0].reshape(rows, ldc)


def oracle_full(p):
    return oracle.gemm(p.A, p.B, p.M, p.N, p.K, p.lda, p.ldb, OLAYOUT[p.layoutA],
                       OLAYOUT[p.layoutB], ODTYPE[p.dtype])


def oracle_rows(p, r0, r1):
    return oracle.gemm_rows(p.A, p.B, p.M, p.N, p.K, p.lda, p.ldb, OLAYOUT[p.layoutA],
                            OLAYOUT[p.layoutB], ODTYPE[p.dtype], r0, r1)


def oracle_entries(p, rows, cols):
    return oracle.gemm_entries(p.A, p.B, p.M, p.N, p.K, p.lda, p.ldb, OLAYOUT[p.layoutA],
                               OLAYOUT[p.layoutB], ODTYPE[p.dtype], rows, cols)


def _pool_map(fn, items):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, min(16, oracle.max_threads()))) as pool:
        return list(pool.map(fn, items))


def oracle_row_set(p, rows):
    """Full rows `rows` of C (len(rows) x N), one single-threaded oracle call
    per row, the calls spread over the host's cores."""
    return np.stack(_pool_map(lambda r: oracle.gemm_rows(
        p.A, p.B, p.M, p.N, p.K, p.lda, p.ldb, OLAYOUT[p.layoutA], OLAYOUT[p.layoutB],
        ODTYPE[p.dtype], int(r), int(r) + 1, threads=1)[0], rows))


def oracle_col_set(p, cols):
    """Full columns `cols` of C (len(cols) x M), as rows of the transposed
    product C^T = B^T A^T: the same bytes read as B^T (A^T) with the layout
    flag B (A) had, which the oracle's transpose pin checks."""
    return np.stack(_pool_map(lambda c: oracle.gemm_rows(
        p.B, p.A, p.N, p.M, p.K, p.ldb, p.lda, OLAYOUT[p.layoutB], OLAYOUT[p.layoutA],
        ODTYPE[p.dtype], int(c), int(c) + 1, threads=1)[0], cols))


def every_tile_rows_cols(M, N, tile=256, seed=0):
    """One row inside every tile row and one column inside every tile column
    of a tile x tile grid, at varying positions within the tile (including
    the tile's first and last), so that every tile has a checked full row and
    a checked full column."""
    rng = np.random.default_rng(seed)
    rows = [min(M - 1, t + (0 if i == 0 else tile - 1 if i == 1 else int(rng.integers(0, tile))))
            for i, t in enumerate(range(0, M, tile))]
    cols = [min(N - 1, t + (tile - 1 if i == 0 else 0 if i == 1 else int(rng.integers(0, tile))))
            for i, t in enumerate(range(0, N, tile))]
    return rows, cols


def gpu_values(C, gdtype):
    """Decoded fp64 values of a GPU output block (numpy)."""
    out = OUT_OF[gdtype]
    if out == "f32":
        return C.astype(np.float64)
    return oracle.decode(C, oracle.BF16 if out == "bf16" else oracle.F16)


def assert_exact(got, ref, gdtype, what=""):
    """Integer-valued case: bit-exact against the exact sum rounded once."""
    out = OUT_OF[gdtype]
    if out == "f32":
        want = ref.astype(np.float32)
        assert np.array_equal(ref, want.astype(np.float64)), "reference not exact in fp32"
        bad = np.nonzero(got.astype(np.float64) != ref)
    else:
        want = oracle.encode(ref, oracle.BF16 if out == "bf16" else oracle.F16)
        bad = np.nonzero(got != want)
    n = bad[0].size
    assert n == 0, f"{what}: {n} mismatches, first at {[int(b[0]) for b in bad]}: " \
                   f"got {got[tuple(b[0] for b in bad)]} want {ref[tuple(b[0] for b in bad)]}"


def tolerance(ref, K, gdtype):
    out = OUT_OF[gdtype]
    if out == "f32":
        return np.full(ref.shape, 1e-5 * K)
    rel = 2.0 ** -8 if out == "bf16" else 2.0 ** -11
    return rel * np.abs(ref) + 1e-5 * K


def assert_close(got, ref, K, gdtype, what=""):
    vals = gpu_values(got, gdtype)
    err = np.abs(vals - ref)
    tol = tolerance(ref, K, gdtype)
    bad = np.nonzero(~(err <= tol))
    n = bad[0].size
    assert n == 0, f"{what}: {n} entries out of tolerance, worst err {np.nanmax(err)}; " \
                   f"first at {[int(b[0]) for b in bad]}"
    return float(np.max(err)) if err.size else 0.0


def assert_canary(C, M, N, gdtype):
    """Everything outside the M x N block must be untouched."""
    canary = CANARY_F32 if OUT_OF[gdtype] == "f32" else CANARY_U16
    outside = np.ones(C.shape, dtype=bool)
    outside[:M, :N] = False
    assert np.all(C[outside] == canary), "C written outside its M x N block"
