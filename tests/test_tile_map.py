"""The workgroup -> tile map (a host build of the kernels' own functions in
lds_layout.h): a bijection onto the tile grid, one contiguous id range per
XCD, the panel reuse it buys in one XCD's round of the 8192^3 launch, and the
per-XCD operand working set that picks the 64 x 64 tile's stage count."""
import ctypes
import os

import pytest

from lds_staged_matrix_amd import build as hip_build


@pytest.fixture(scope="module")
def lib():
    path = hip_build.layout_host_path("")
    if not os.path.exists(path):
        hip_build.build_layout_host()
    lib = ctypes.CDLL(path)
    lib.lsm_xcd_logical_id.restype = ctypes.c_int
    lib.lsm_xcd_logical_id.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.lsm_tile_coords.restype = None
    lib.lsm_tile_coords.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_int)] * 2
    lib.lsm_xcd_max_panel_bytes.restype = ctypes.c_longlong
    lib.lsm_xcd_max_panel_bytes.argtypes = [ctypes.c_int] * 3 + [ctypes.c_longlong] * 2
    return lib


def coords(lib, lid, tiles_m, tiles_n, group_m):
    tm, tn = ctypes.c_int(), ctypes.c_int()
    lib.lsm_tile_coords(lid, tiles_m, tiles_n, group_m, ctypes.byref(tm), ctypes.byref(tn))
    return tm.value, tn.value


@pytest.mark.parametrize("nwg", [1, 5, 7, 8, 9, 64, 255, 256, 1000, 1023, 1024, 4097])
def test_xcd_logical_id_is_a_bijection_with_contiguous_ranges_per_xcd(lib, nwg):
    ids = [lib.lsm_xcd_logical_id(b, nwg) for b in range(nwg)]
    assert sorted(ids) == list(range(nwg))
    for x in range(8):
        mine = [ids[b] for b in range(x, nwg, 8)]          # workgroups on XCD x, in order
        assert mine == list(range(mine[0], mine[0] + len(mine))) if mine else True


@pytest.mark.parametrize("tiles_m,tiles_n,group_m", [(32, 32, 8), (16, 16, 8), (12, 9, 8),
                                                     (1, 256, 8), (47, 18, 8), (5, 3, 4),
                                                     (9, 7, 16)])
def test_tile_coords_cover_the_grid_once(lib, tiles_m, tiles_n, group_m):
    seen = {coords(lib, l, tiles_m, tiles_n, group_m) for l in range(tiles_m * tiles_n)}
    assert seen == {(m, n) for m in range(tiles_m) for n in range(tiles_n)}


def test_one_xcd_round_of_the_8192_launch_shares_panels(lib):
    # 8192^3 with 256 x 256 tiles: 32 x 32 tiles, 256 CUs (32 per XCD) run
    # the first 256 workgroups together.  With the map, the 32 workgroups of
    # each XCD hold an 8 x 4 block of tiles: 8 A panels + 4 B panels reach its
    # L2.  In hardware order the same 32 workgroups would hold one tile row
    # spread over 32 columns: 1 + 32 panels.
    nwg, tiles = 1024, 32
    for x in range(8):
        tl = [coords(lib, lib.lsm_xcd_logical_id(x + 8 * j, nwg), tiles, tiles, 8) for j in range(32)]
        assert len({m for m, _ in tl}) == 8 and len({n for _, n in tl}) == 4
        hw = [coords(lib, x + 8 * j, tiles, tiles, 8) for j in range(32)]
        assert len({m for m, _ in hw}) + len({n for _, n in hw}) == 33


def brute_xcd_panels(lib, tiles_m, tiles_n, group_m, a_panel, b_panel):
    """Largest A + B panel bytes over the 8 XCDs, counted tile by tile: workgroup
    b runs on XCD b mod 8 and computes tile_coords(xcd_logical_id(b))."""
    nwg = tiles_m * tiles_n
    rows = [set() for _ in range(8)]
    cols = [set() for _ in range(8)]
    for b in range(nwg):
        tm, tn = coords(lib, lib.lsm_xcd_logical_id(b, nwg), tiles_m, tiles_n, group_m)
        rows[b & 7].add(tm)
        cols[b & 7].add(tn)
    return max(len(r) * a_panel + len(c) * b_panel for r, c in zip(rows, cols))


@pytest.mark.parametrize("tiles_m", [1, 2, 3, 7, 8, 9, 13, 16, 17, 24, 33])
@pytest.mark.parametrize("tiles_n", [1, 2, 5, 8, 9, 16, 18, 31])
def test_xcd_max_panel_bytes_matches_brute_force(lib, tiles_m, tiles_n):
    # distinct weights for A and B panels, so a swapped row/column count shows
    got = lib.lsm_xcd_max_panel_bytes(tiles_m, tiles_n, 8, 1000, 1)
    assert got == brute_xcd_panels(lib, tiles_m, tiles_n, 8, 1000, 1)


@pytest.mark.parametrize("M,N,K,panels,four", [
    (512, 512, 3072, 9, False),      # 8 rows x 1 column per XCD: 3.5 MiB, fits the 4 MiB L2
    (512, 512, 4096, 9, True),       # 4.7 MB: four stages
    (1024, 1024, 2048, 12, False),   # 8 rows x 4 columns: 3.1 MB
    (1024, 1024, 3072, 12, True),
    (1500, 1152, 896, 24, False),    # ranges straddle two groups of tile rows: 16 + 8 panels
    (1500, 1152, 1792, 24, True),
])
def test_stage_rule_on_measured_shapes(lib, M, N, K, panels, four):
    """The panel counts behind the 64 x 64 tile's choice of four LDS stages
    (panel = 64 rows x K bf16), on the shapes it was measured on."""
    tm, tn = -(-M // 64), -(-N // 64)
    one = lib.lsm_xcd_max_panel_bytes(tm, tn, 8, 1, 1)
    assert one == panels
    assert (panels * 64 * K * 2 > 4 << 20) == four
