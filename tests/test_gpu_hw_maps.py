"""The hardware maps the kernels rely on, checked one at a time on the GPU
against the CPU formulas of lds_layout.h / gemm_common.h (through the
host-only build of the layout functions) with the probe kernels of
libhw_probe.so.

* Fragment reads.  The host lays out an LDS tile image with the library's
  layout functions (each element holds a tag naming its logical row and k);
  the probe reads every fragment of the tile with the library's own device
  read functions -- ds_read_b128 for K-contiguous tiles, ds_read_b64_tr_b16
  and ds_read_b64_tr_b8 for MN-contiguous ones ("Lds Optimization", "MFMA
  Transpose Load from LDS (gfx950 only)") -- and every lane must hold exactly
  the elements of the MFMA operand layout:
    32x32x16:  lane l, element i: row/column l & 31, k = 16 kk + 8 (l >> 5) + i
    16x16x32:  lane l, element i: row/column l & 15, k = 32 kk + 8 (l >> 4) + i
    32x32x64 (E4M3): lane l, byte b: row/column l & 31, k = 64 kk + 32 (l >> 5) + b
    16x16x128 (E4M3): lane l, byte b: row/column l & 15,
                      k = 128 kk + 16 ((l >> 4) + 4 (b >> 4)) + (b & 15)
  This pins the transposed reads' lane exchange together with the address
  functions that rely on it.
* MFMA layouts.  One MFMA on operands placed by those layouts must give
  A @ B placed by the accumulator layouts (AccLayout in gemm_common.h):
    32 x 32: register r of lane l = C[8 (r >> 2) + 4 (l >> 5) + (r & 3)][l & 31]
    16 x 16: register r of lane l = C[4 (l >> 4) + r][l & 15]
  on random integers (exact in fp32) and on one-hot inputs.  Which k slot of
  a lane pairs with which is not observable through a product as long as A
  and B use the same numbering, and the kernels always do.
* The buffer range check of the direct-to-LDS loads: a 16-byte load through
  a buffer resource of N bytes returns zeros when its vector offset plus its
  scalar offset reaches past N, even when the vector offset alone is in
  range; the kernels carry the K advance and the load round in the scalar
  offset and rely on this for the rows past K, M or N of edge tiles.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from lds_staged_matrix_amd import build as hip_build

pytestmark = pytest.mark.gpu

KINDS = {
    # name: (kind id, K-contiguous?, rows of the stored tile, row bytes, element bytes, mfma)
    "KC256": (0, True, 256, 128, 2, 32),
    "KC64x128": (1, True, 64, 256, 2, 32),
    "MN256": (2, False, 64, 512, 2, 32),
    "MN128": (3, False, 64, 256, 2, 32),
    "MN64": (4, False, 64, 128, 2, 32),
    "MN256_16": (5, False, 64, 512, 2, 16),
    "KC256_16": (6, True, 256, 128, 2, 16),
    "KC8": (7, True, 256, 128, 1, 32),
    "MN8": (8, False, 128, 256, 1, 32),
    "MN8_128": (9, False, 128, 128, 1, 32),
    "KC8_16": (10, True, 256, 128, 1, 16),
    "MN8_16": (11, False, 128, 256, 1, 16),
}


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib = ctypes.CDLL(hip_build.HW_PROBE)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.lsm_probe_frag.argtypes = [i32, vp, i32, i32, i32, vp, vp]
    lib.lsm_probe_mfma.argtypes = [i32, i32, vp, vp, vp, vp]
    lib.lsm_probe_range.argtypes = [vp, ctypes.c_uint32, ctypes.c_uint32, vp, vp, vp]
    lib.lsm_probe_pad.argtypes = [i32, i32, vp, vp]
    for f in ("lsm_probe_frag", "lsm_probe_mfma", "lsm_probe_range", "lsm_probe_pad"):
        getattr(lib, f).restype = i32
    return lib


@pytest.fixture(scope="module")
def layout():
    lib = ctypes.CDLL(hip_build.layout_host_path(""))
    for f in ("lsm_kc_chunk_offset", "lsm_mn_chunk_offset", "lsm_mn16_chunk_offset",
              "lsm_mn_chunk_offset8", "lsm_mn16_chunk_offset8"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def stream():
    return torch.cuda.current_stream().cuda_stream


def tile_image(layout, kc, rows, rb, es, mf16, tag_of):
    """The LDS image of a tile: logical element (outer row r, inner e) at the
    place the library's layout functions give it, holding tag_of(r, e)."""
    img = np.zeros(rows * rb // es, dtype=np.uint16 if es == 2 else np.uint8)
    epc = 16 // es
    for r in range(rows):
        for c in range(rb // 16):
            if kc:
                off = layout.lsm_kc_chunk_offset(r, c, rb)
            elif mf16:
                off = layout.lsm_mn16_chunk_offset(r, c, rb) if es == 2 else \
                    layout.lsm_mn16_chunk_offset8(r, c, rb)
            elif es == 1:
                off = layout.lsm_mn_chunk_offset8(r, c, rb)
            else:
                off = layout.lsm_mn_chunk_offset(r, c, rb)
            for e in range(epc):
                img[off // es + e] = tag_of(r, c * epc + e)
    return img


@pytest.mark.parametrize("name", sorted(KINDS))
def test_fragment_reads_deliver_the_mfma_operand_layout(probe, layout, name):
    kind, kc, rows, rb, es, mf = KINDS[name]
    inner = rb // es
    # operand rows/columns of the tile (M or N extent) and its K extent
    mn, bk = (rows, inner) if kc else (inner, rows)
    # tag of operand element (row/column x, k): x * bk + k, below 2^15
    if kc:
        tag = lambda r, e: r * bk + e          # outer = x, inner = k
    else:
        tag = lambda r, e: e * bk + r          # outer = k, inner = x
    passes = [0] if es == 2 else [0, 1]        # one-byte elements: low, then high tag byte
    fw = 16 if mf == 16 else 32               # fragment width
    kstep = {(2, 32): 16, (2, 16): 32, (1, 32): 64, (1, 16): 128}[(es, mf)]
    per_lane = 8 if es == 2 else 32
    print(f"CASE fragment reads {name}", flush=True)
    got = {}
    for ps in passes:
        t = (lambda r, e: tag(r, e)) if es == 2 else (lambda r, e, ps=ps: (tag(r, e) >> (8 * ps)) & 0xFF)
        img = tile_image(layout, kc, rows, rb, es, mf == 16, t)
        dimg = torch.from_numpy(img.view(np.uint8).copy()).cuda()
        out = torch.zeros(64 * 32, dtype=torch.uint8, device="cuda")
        for base in range(0, mn, fw):
            for kk in range(bk // kstep):
                st = probe.lsm_probe_frag(kind, dimg.data_ptr(), img.nbytes, base, kk, out.data_ptr(),
                                          stream())
                assert st == 0
                torch.cuda.synchronize()
                v = out.cpu().numpy()
                v = v[:64 * 16].view(np.uint16).reshape(64, 8) if es == 2 else v.reshape(64, 32)
                got.setdefault((base, kk), 0)
                got[(base, kk)] = got[(base, kk)] + (v.astype(np.int64) << (8 * ps))
    for (base, kk), v in got.items():
        for l in range(64):
            x = base + (l & (fw - 1))
            if (es, mf) == (1, 16):
                # 16x16x128: byte b of group g is k = 16 (g + 4 (b >> 4)) + (b & 15)
                ks = [kstep * kk + 16 * ((l >> 4) + 4 * (b >> 4)) + (b & 15) for b in range(32)]
            else:
                k0 = kstep * kk + (per_lane if es == 2 else 32) * (l // fw)
                ks = [k0 + i for i in range(per_lane)]
            want = [x * bk + k for k in ks]
            assert list(v[l]) == want, (name, base, kk, l)


BF16 = {-2: 0xC000, -1: 0xBF80, 0: 0, 1: 0x3F80, 2: 0x4000}
F16 = {-2: 0xC000, -1: 0xBC00, 0: 0, 1: 0x3C00, 2: 0x4000}
E4M3 = {-2: 0xC0, -1: 0xB8, 0: 0, 1: 0x38, 2: 0x40}


def run_mfma(probe, shape, in_type, A, B):
    """Place A (rows x k) and B (k x cols) into lane registers by the operand
    layout, run one MFMA, read C back by the accumulator layout."""
    enc = {0: BF16, 1: F16, 2: E4M3}[in_type]
    kpl = 32 if in_type == 2 else 8                       # k per lane
    groups = 64 // shape
    if in_type == 2:
        a = np.zeros((64, 32), np.uint8)
        b = np.zeros((64, 32), np.uint8)
    else:
        a = np.zeros((64, 8), np.uint16)
        b = np.zeros((64, 8), np.uint16)
    for l in range(64):
        x, g = l % shape, l // shape
        for i in range(kpl):
            a[l, i] = enc[int(A[x, kpl * g + i])]
            b[l, i] = enc[int(B[kpl * g + i, x])]
    da = torch.from_numpy(a.view(np.uint8).copy()).cuda()
    db = torch.from_numpy(b.view(np.uint8).copy()).cuda()
    regs = 16 if shape == 32 else 4
    out = torch.zeros(regs * 64, dtype=torch.float32, device="cuda")
    assert probe.lsm_probe_mfma(shape, in_type, da.data_ptr(), db.data_ptr(), out.data_ptr(),
                                stream()) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(regs, 64)
    C = np.full((shape, shape), np.nan)
    for r in range(regs):
        for l in range(64):
            row = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3) if shape == 32 else 4 * (l >> 4) + r
            col = l % shape
            assert np.isnan(C[row, col]), "accumulator layout maps two registers to one entry"
            C[row, col] = o[r, l]
    return C


MFMAS = [(32, 0), (32, 1), (16, 0), (16, 1), (32, 2), (16, 2)]     # (shape, input type)
DEPTH = {(32, 0): 16, (32, 1): 16, (16, 0): 32, (16, 1): 32, (32, 2): 64, (16, 2): 128}


@pytest.mark.parametrize("shape,in_type", MFMAS)
def test_mfma_layouts_random_integers(probe, shape, in_type):
    K = DEPTH[(shape, in_type)]
    rng = np.random.default_rng(100 + shape + in_type)
    print(f"CASE mfma {shape} input {in_type} random", flush=True)
    for _ in range(3):
        A = rng.integers(-2, 3, size=(shape, K))
        B = rng.integers(-2, 3, size=(K, shape))
        C = run_mfma(probe, shape, in_type, A, B)
        assert np.array_equal(C, (A @ B).astype(np.float64))


@pytest.mark.parametrize("shape,in_type", [(32, 0), (16, 0), (32, 2), (16, 2)])
def test_mfma_layouts_one_hot(probe, shape, in_type):
    # A = e(i, k), B = e(k, j): C must be 1 at (i, j) and 0 elsewhere
    K = DEPTH[(shape, in_type)]
    rng = np.random.default_rng(7)
    print(f"CASE mfma {shape} input {in_type} one-hot", flush=True)
    for i, k, j in [(0, 0, 0), (shape - 1, K - 1, shape - 1)] + \
                   [tuple(int(x) for x in rng.integers(0, [shape, K, shape])) for _ in range(6)]:
        A = np.zeros((shape, K), np.int64)
        B = np.zeros((K, shape), np.int64)
        A[i, k] = 1
        B[k, j] = 1
        C = run_mfma(probe, shape, in_type, A, B)
        want = np.zeros((shape, shape))
        want[i, j] = 1
        assert np.array_equal(C, want), (i, k, j)


# (num_records, scalar offset): chunk l (vector offset 16 l) must read data iff
# 16 l + soffset + 16 <= num_records.  The allocation behind the buffer is
# 32 KiB, so every access stays inside it whatever the hardware does.
RANGE_CASES = [(4096, 0), (4096, 3072), (4096, 3584), (4096, 4096), (4096, 8192),
               (1536, 1024), (512, 0), (8192, 7680), (4096, 16384)]


@pytest.mark.parametrize("num_records,soff", RANGE_CASES)
def test_buffer_range_check_covers_the_scalar_offset(probe, num_records, soff):
    print(f"CASE buffer range num_records {num_records} soffset {soff}", flush=True)
    words = 8192
    assert 16 * 64 + soff <= 4 * words
    buf = torch.arange(words, dtype=torch.int64, device="cuda").to(torch.int32) + 0x10000000
    out_reg = torch.zeros(256, dtype=torch.int32, device="cuda")
    out_lds = torch.zeros(256, dtype=torch.int32, device="cuda")
    assert probe.lsm_probe_range(buf.data_ptr(), num_records, soff, out_reg.data_ptr(),
                                 out_lds.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    for name, o in (("registers", out_reg), ("direct-to-LDS", out_lds)):
        v = o.cpu().numpy().reshape(64, 4)
        for l in range(64):
            start = 16 * l + soff
            want = host[start // 4:start // 4 + 4] if start + 16 <= num_records else np.zeros(4)
            assert np.array_equal(v[l], want), (name, l, v[l], want)


def test_padded_column_probe_runs(probe):
    # the counter-calibration probe of the padding table: every pad runs and
    # returns the sum of the zeros it read
    out = torch.full((1,), 7.0, device="cuda")
    for pad in (0, 1, 2, 4, 32):
        assert probe.lsm_probe_pad(pad, 100, out.data_ptr(), stream()) == 0
        torch.cuda.synchronize()
        assert float(out.item()) == 0.0
    assert probe.lsm_probe_pad(3, 100, out.data_ptr(), stream()) == -1


def test_lane_address_read_probe_runs_and_refuses_bad_addresses(probe):
    # the bank-pass probe of ds_read_b64 / _tr_b8 / _b128: every mode runs on
    # in-range addresses and returns the fold of what it read; addresses out
    # of range or misaligned are refused on the host with nothing launched
    probe.lsm_probe_lds_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
    probe.lsm_probe_lds_read.restype = ctypes.c_int
    out = torch.zeros(64, dtype=torch.int32, device="cuda")
    for mode, width in ((0, 8), (1, 8), (2, 16)):
        good = (ctypes.c_int * 64)(*[width * l for l in range(64)])
        assert probe.lsm_probe_lds_read(mode, good, 3, out.data_ptr(), stream()) == 0
        torch.cuda.synchronize()
        if mode == 0:
            # LDS holds dword i at byte 4 i; lane l folds (2 l) ^ (2 l + 1) = 1, three times
            assert out.cpu().tolist() == [3] * 64
    for bad in ([65536 - 8] + [0] * 63, [4] + [0] * 63, [-16] + [0] * 63):
        arr = (ctypes.c_int * 64)(*bad)
        assert probe.lsm_probe_lds_read(2, arr, 3, out.data_ptr(), stream()) == -1
    assert probe.lsm_probe_lds_read(3, (ctypes.c_int * 64)(), 3, out.data_ptr(), stream()) == -1
