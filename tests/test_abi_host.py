"""Host-side checks of the C ABI library: loading, exported symbols, argument
validation (no GPU needed: every check happens before the first HIP call),
the tile scheduler's mapping and the measurement formulas."""
import ctypes
import os
import re

import numpy as np
import pytest

import gemv_tile_pipelined_amd as gt
from gemv_tile_pipelined_amd import metrics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemvtile.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

OK, INVALID, UNSUPPORTED = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gt.LIBRARY_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return gt.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(gt.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(6):
        assert gt.status_string(code)
    assert gt.status_string(99) == "unknown status"


def _gemm(lib, A, B, D, M, N, K):
    return lib.gemm_f16(A, B, D, M, N, K, None)


def _gemv(lib, x, W, y, N, K):
    return lib.gemv_f16(x, W, y, N, K, None)


FAKE = 0x10000  # a 16-byte aligned address; never dereferenced by these calls
# The split-K rule's constants as the header documents them: K tiles of 64
# per slice at least; K tiles the split must take off the K loop, plus one
# per SPLITK_OUTPUTS_PER_TILE partial sums.
SPLITK_MIN_TILES = 10
SPLITK_MIN_SAVED = 12
SPLITK_OUTPUTS_PER_TILE = 262144


def test_gemm_argument_validation(lib):
    assert _gemm(lib, FAKE, FAKE, FAKE, -1, 4, 8) == INVALID
    assert _gemm(lib, FAKE, FAKE, FAKE, 4, -1, 8) == INVALID
    assert _gemm(lib, FAKE, FAKE, FAKE, 4, 4, -8) == INVALID
    assert _gemm(lib, FAKE, FAKE, None, 4, 4, 8) == INVALID
    assert _gemm(lib, None, FAKE, FAKE, 4, 4, 8) == INVALID
    assert _gemm(lib, FAKE, None, FAKE, 4, 4, 8) == INVALID
    # empty outputs are a no-op, even with NULL pointers
    assert _gemm(lib, None, None, None, 0, 4, 8) == OK
    assert _gemm(lib, None, None, None, 4, 0, 8) == OK
    # K must be a multiple of 8; A/B 16-byte aligned; D 2-byte aligned
    assert _gemm(lib, FAKE, FAKE, FAKE, 4, 4, 12) == UNSUPPORTED
    assert _gemm(lib, FAKE + 8, FAKE, FAKE, 4, 4, 8) == UNSUPPORTED
    assert _gemm(lib, FAKE, FAKE + 2, FAKE, 4, 4, 8) == UNSUPPORTED
    assert _gemm(lib, FAKE, FAKE, FAKE + 1, 4, 4, 8) == UNSUPPORTED
    # size limits
    assert _gemm(lib, FAKE, FAKE, FAKE, 4, 4, 4194304) == UNSUPPORTED
    assert _gemm(lib, FAKE, FAKE, FAKE, 2**31, 4, 8) == UNSUPPORTED
    # unknown internal variant: each family has its own id range (tiled 0..,
    # skinny 100.., wave-specialised 200..); the gaps, and the numbers of
    # ablations measured and not kept, are invalid
    for bad in (-1, 4, 9, 11, 12, 15, 19, 29, 33, 36, 99, 101, 113, 131, 140, 148, 149, 153, 199, 202, 1000):
        assert lib.gemvtile_gemm_f16_variant(FAKE, FAKE, FAKE, 4, 4, 8, None, bad) == INVALID, bad
    # skinny launch shapes only apply when one side has at most 16 rows (at
    # most 64 for gemm_f16's own skinny launch, 100, and the small-side
    # split, 160)
    for v in (104, 112, 130, 147, 152):
        assert lib.gemvtile_gemm_f16_variant(FAKE, FAKE, FAKE, 32, 32, 8, None, v) == UNSUPPORTED, v
    for v in (100, 160):
        assert lib.gemvtile_gemm_f16_variant(FAKE, FAKE, FAKE, 65, 65, 8, None, v) == UNSUPPORTED, v


def test_gemm_bias_argument_validation(lib):
    """gemm_bias_f16 / gemm_bias_bf16: the GEMM checks, then the activation
    code and the bias pointer, all before any HIP call."""
    for fn in (lib.gemm_bias_f16, lib.gemm_bias_bf16):
        # act must be NONE (0) or RELU (1), even for an empty output
        for bad in (-1, 2, 7):
            assert fn(FAKE, FAKE, FAKE, FAKE, 4, 4, 8, bad, None) == INVALID, bad
            assert fn(None, None, None, None, 0, 4, 8, bad, None) == INVALID, bad
        # the GEMM's own checks
        assert fn(FAKE, FAKE, FAKE, FAKE, -1, 4, 8, 0, None) == INVALID
        assert fn(FAKE, FAKE, FAKE, None, 4, 4, 8, 0, None) == INVALID
        assert fn(None, FAKE, FAKE, FAKE, 4, 4, 8, 1, None) == INVALID
        assert fn(FAKE, FAKE, FAKE, FAKE, 4, 4, 12, 0, None) == UNSUPPORTED
        assert fn(FAKE + 8, FAKE, FAKE, FAKE, 4, 4, 8, 0, None) == UNSUPPORTED
        # empty outputs are a no-op, with or without a bias
        assert fn(None, None, None, None, 0, 4, 8, 1, None) == OK
        assert fn(None, None, FAKE, None, 4, 0, 8, 0, None) == OK
        # the bias must be element aligned (NULL is allowed: no bias)
        assert fn(FAKE, FAKE, FAKE + 1, FAKE, 4, 4, 8, 0, None) == UNSUPPORTED


def test_gemv_argument_validation(lib):
    assert _gemv(lib, FAKE, FAKE, FAKE, -1, 8) == INVALID
    assert _gemv(lib, FAKE, FAKE, FAKE, 4, -8) == INVALID
    assert _gemv(lib, FAKE, FAKE, None, 4, 8) == INVALID
    assert _gemv(lib, None, FAKE, FAKE, 4, 8) == INVALID
    assert _gemv(lib, FAKE, None, FAKE, 4, 8) == INVALID
    assert _gemv(lib, None, None, None, 0, 8) == OK
    assert _gemv(lib, FAKE, FAKE, FAKE, 4, 9) == UNSUPPORTED
    assert _gemv(lib, FAKE + 4, FAKE, FAKE, 4, 8) == UNSUPPORTED
    assert _gemv(lib, FAKE, FAKE + 8, FAKE, 4, 8) == UNSUPPORTED
    assert _gemv(lib, FAKE, FAKE, FAKE + 1, 4, 8) == UNSUPPORTED
    for bad in (-1, 1, 5, 13, 17, 19, 22, 27, 30, 36, 42, 99):
        assert lib.gemvtile_gemv_f16_variant(FAKE, FAKE, FAKE, 4, 8, None, bad) == INVALID, bad


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(gt.GemvTileLibraryMissing):
        gt.load_library(str(tmp_path / "missing.so"))


def _tile_counts():
    out = {}
    for line in open(os.path.join(GOLDEN, "tile_counts.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            out[k] = int(v)
    return out


@pytest.mark.parametrize(
    "M,N",
    [(256, 256), (4096, 4096), (4000, 4032), (8192, 8192), (257, 255), (2304, 4096), (100, 9000), (4096, 128)],
)
def test_grouped_order_is_a_bijection(lib, M, N):
    cfg = gt.gemm_config()
    tiles_m = -(-M // cfg["BM"])
    tiles_n = -(-N // cfg["BN"])
    seen = set()
    for t in range(tiles_m * tiles_n):
        tm, tn = gt.tile_coord(t, tiles_m, tiles_n, cfg["group_m"])
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == tiles_m * tiles_n


def test_grouped_order_shape(lib):
    # Inside a full group the index runs down group_m tile rows of one column,
    # then moves to the next column; the last group may be shorter.
    assert [gt.tile_coord(t, 16, 16, 8) for t in range(10)] == [(r, 0) for r in range(8)] + [(0, 1), (1, 1)]
    # tiles_m = 10 with group_m = 8: the second group is 2 rows high
    assert [gt.tile_coord(t, 10, 3, 8) for t in range(24, 30)] == [(8, 0), (9, 0), (8, 1), (9, 1), (8, 2), (9, 2)]


def test_tile_coord_large_grids():
    """Grids of 2^30 tiles or more take the 64-bit form of the mapping; near
    that size both forms must stay in range and one-to-one (sampled), and
    the first group runs down its 8 tile rows."""
    rng = np.random.default_rng(7)
    for tiles_m, tiles_n in ((1 << 15, (1 << 15) - 1), (1 << 15, (1 << 15) + 3), (8, 1 << 27), (3, 1 << 23)):
        total = tiles_m * tiles_n
        ts = np.unique(np.concatenate([rng.integers(0, total, 2000), [0, 1, total - 2, total - 1]]))
        coords = [gt.tile_coord(int(t), tiles_m, tiles_n, 8) for t in ts]
        assert all(0 <= tm < tiles_m and 0 <= tn < tiles_n for tm, tn in coords)
        assert len(set(coords)) == len(coords)
        rows = min(8, tiles_m)
        assert [gt.tile_coord(t, tiles_m, tiles_n, 8) for t in range(rows + 1)] == \
            [(r, 0) for r in range(rows)] + [(0, 1)]


def test_tile_coord_rejects_bad_input(lib):
    tm, tn = ctypes.c_int64(), ctypes.c_int64()
    assert lib.gemvtile_tile_coord(16, 4, 4, 8, ctypes.byref(tm), ctypes.byref(tn)) == INVALID
    assert lib.gemvtile_tile_coord(-1, 4, 4, 8, ctypes.byref(tm), ctypes.byref(tn)) == INVALID
    assert lib.gemvtile_tile_coord(0, 0, 4, 8, ctypes.byref(tm), ctypes.byref(tn)) == INVALID
    assert lib.gemvtile_tile_coord(0, 4, 4, 0, ctypes.byref(tm), ctypes.byref(tn)) == INVALID
    assert lib.gemvtile_tile_coord(0, 4, 4, 8, None, ctypes.byref(tn)) == INVALID


@pytest.mark.parametrize("grid", [1, 7, 8, 64, 200, 256, 1024])
def test_xcd_renumbering_is_a_bijection(lib, grid):
    ids = [gt.xcd_logical_id(w, grid) for w in range(grid)]
    assert sorted(ids) == list(range(grid))
    if grid % 8 == 0:
        # workgroup w runs on XCD w % 8; each XCD owns one contiguous id range
        per = grid // 8
        for w in range(grid):
            assert ids[w] // per == w % 8
    assert gt.xcd_logical_id(grid, grid) == -1


def test_gemm_grid_and_golden_counts(lib):
    cfg = gt.gemm_config()
    assert cfg == {"BM": 256, "BN": 256, "BK": 64, "stages": 2, "threads": 256, "group_m": 8}
    assert gt.gemm_grid(4096, 4096, 4096, 256) == 256
    assert gt.gemm_grid(8192, 8192, 4096, 256) == 256
    assert gt.gemm_grid(256, 256, 4096, 256) == 8  # eight 128x64 tiles (see the tile rule below)
    assert gt.gemm_grid(4000, 4032, 4096, 256) == 256
    assert gt.gemm_grid(0, 4, 4096, 256) == 0
    # skinny shapes: from 32 rows of the larger side per CU, one workgroup
    # per 32, 48 or 64 rows (the fewest rows per CU over whole rounds of
    # workgroups, ties to the larger), else per 16, 8, 4, 2 or 1 rows
    assert gt.gemm_grid(8, 4096, 4096, 256) == 256
    assert gt.gemm_grid(4096, 16, 4096, 256) == 256
    assert gt.gemm_grid(8, 8192, 4096, 256) == 256  # 32 rows per workgroup
    assert gt.gemm_grid(8, 8191, 4096, 256) == 512  # 16 rows per workgroup
    assert gt.gemm_grid(8, 10300, 4096, 256) == 215  # 48 rows: one round
    assert gt.gemm_grid(64, 14400, 4096, 256) == 225  # 64 rows: one round
    assert gt.gemm_grid(16400, 40, 4096, 256) == 342  # 48 rows: 96 per CU, as with 32
    assert gt.gemm_grid(8, 3000, 4096, 256) == 375
    assert gt.gemm_grid(8, 2000, 4096, 256) == 500
    assert gt.gemm_grid(1000, 9, 4096, 256) == 500
    assert gt.gemm_grid(16, 300, 4096, 256) == 300
    assert gt.gemm_grid(16, 16, 4096, 256) == 16
    # 17..64 rows on the smaller side: the skinny kernel too, over the larger side
    assert gt.gemm_grid(17, 4097, 4096, 256) == 257  # 16 rows per workgroup
    # ... with the small side split into 16-row blocks (grid y) where the
    # staged launch would take fewer than 8 rows per workgroup, or 8 with at
    # most 32 small-side rows: blocks x workgroups of the most of 16, 8, 4, 2
    # rows that still give every CU one
    assert gt.gemm_grid(32, 1000, 4096, 256) == 2 * 250  # 4 rows per workgroup
    assert gt.gemm_grid(4000, 30, 4096, 256) == 2 * 250  # 16 rows per workgroup
    assert gt.gemm_grid(20, 24, 4096, 256) == 2 * 24  # 1 row per workgroup
    assert gt.gemm_grid(64, 1024, 14336, 256) == 4 * 64
    assert gt.gemm_grid(1500, 48, 4104, 256) == 3 * 94
    assert gt.gemm_grid(30, 2100, 4096, 256) == 2 * 132  # staged: 8 rows, at most 32 small-side rows
    assert gt.gemm_grid(50, 2100, 4096, 256) == 263  # staged, 8 rows per workgroup
    assert gt.gemm_grid(64, 4097, 4096, 256) == 257
    assert gt.gemm_grid(65, 4097, 4096, 256) == 65  # 1 x 65 tiles of 128x64
    # ... whatever the larger side
    assert gt.gemm_grid(32, 16384, 4096, 256) == 256  # 64 rows per workgroup
    assert gt.gemm_grid(24, 8192, 4096, 256) == 256
    assert gt.gemm_grid(24, 16384, 4096, 256) == 256
    assert gt.gemm_grid(20, 12288, 4096, 256) == 256  # 48 rows per workgroup
    assert gt.gemm_grid(20, 12289, 4096, 256) == 193  # 64 rows: 64 per CU, as with 32
    assert gt.gemm_grid(8191, 17, 4096, 256) == 512
    assert gt.gemm_grid(33, 8192, 4096, 256) == 256
    assert gt.gemm_grid(16, 8192, 4096, 256) == 256
    assert gt.gemm_grid(32, 16385, 4096, 256) == 342
    assert gt.gemm_grid(64, 8192, 4096, 256) == 256
    assert gt.gemm_grid(14336, 64, 4096, 256) == 224
    assert gt.gemm_grid(65536, 64, 4096, 256) == 1024
    assert gt.gemm_grid(65536, 65, 4096, 256) == 256  # tiled
    # one row on a side: the GEMV grid of the other side
    assert gt.gemm_grid(1, 4096, 4096, 256) == gt.gemv_grid(4096, 4096, 256) == 256
    assert gt.gemm_grid(1000, 1, 4096, 256) == gt.gemv_grid(1000, 4096, 256)
    assert gt.gemm_grid(1, 4096, 14336, 256) == gt.gemv_grid(4096, 14336, 256) == 2048
    golden = _tile_counts()
    # The TVM chapter's counts at its 128x128 tiles and BLK_K = 64: the same
    # tile-count arithmetic, applied to its parameters.
    assert -(-4096 // 128) * -(-4096 // 128) == golden["tiles_4096x4096_at_128x128"]
    assert 4096 // 64 == golden["k_iterations_k4096_bk64"]
    assert golden["k_iterations_k4096_bk64"] // 2 == golden["uses_per_stage_depth2"]
    assert 128 * 64 * metrics.FP16_BYTES == golden["tile_bytes_128x64"]
    assert (128 * 64 + 128 * 64) * metrics.FP16_BYTES == golden["stage_bytes_128x64_pair"]
    # every output tile visited once: 1024 tiles at 128x128 for 4096^2
    seen = {gt.tile_coord(t, 32, 32, 8) for t in range(1024)}
    assert len(seen) == golden["tiles_4096x4096_at_128x128"]


def test_gemm_tile_rule(lib):
    """The tiled GEMM's tile: 256x256 while it fills the CUs, smaller tiles
    (with deeper rings) when it would not.  The shapes are those the choice
    was measured on; the last two differ only in orientation."""
    want = {
        (4096, 4096): (256, 256, 2),
        (8192, 8192): (256, 256, 2),
        (4000, 4032): (256, 256, 2),
        (8192, 1024): (256, 128, 3),
        (4096, 2048): (256, 128, 3),
        (2048, 2048): (128, 128, 4),
        (1024, 4096): (128, 128, 4),
        (512, 4096): (128, 64, 4),
        (256, 256): (128, 64, 4),
        (1024, 1024): (128, 64, 4),
        (1536, 1024): (128, 64, 4),
        (2176, 3840): (128, 256, 3),
        (3840, 2176): (256, 128, 3),
    }
    for (M, N), tile in want.items():
        assert gt.gemm_tile(M, N, 256) == tile, (M, N)
        bm, bn, _ = tile
        assert gt.gemm_grid(M, N, 4096, 256) == min(-(-M // bm) * -(-N // bn), 256), (M, N)
    # the documented cost, ceil(#tiles / CUs) * bm * bn / rate, is least for
    # the chosen tile, and no larger tile ties it
    shapes = [(bm, bn, st, rate) for bm, bn, st, rate in
              ((256, 256, 2, 1.0), (256, 128, 3, 0.9), (128, 256, 3, 0.9), (128, 128, 4, 0.76),
               (128, 64, 4, 0.55))]
    for M in (17, 100, 256, 300, 777, 1024, 2049, 4096, 6000):
        for N in (17, 129, 512, 1000, 3000, 8192):
            for cus in (80, 256, 304):
                cost = [-(-(-(-M // bm) * -(-N // bn)) // cus) * bm * bn / rate for bm, bn, _, rate in shapes]
                got = gt.gemm_tile(M, N, cus)
                i = [s[:3] for s in shapes].index(got)
                assert cost[i] <= min(cost) * (1 + 1e-12), (M, N, cus)
                assert all(c > cost[i] * (1 + 1e-12) for c in cost[:i]), (M, N, cus)
    for bad in ((0, 4, 256), (4, 0, 256), (4, 4, 0), (4, 4, 2**21)):
        with pytest.raises(gt.GemvTileError):
            gt.gemm_tile(*bad)


def _splitk_tile(M, N, cus):
    # split K picks by the same cost as gemm_tile among the first four
    # tiles (256x256, 256x128, 128x256, 128x128), ties to the larger
    shapes = ((256, 256, 1.0), (256, 128, 0.9), (128, 256, 0.9), (128, 128, 0.76))
    cost = [-(-(-(-M // bm) * -(-N // bn)) // cus) * bm * bn / rate for bm, bn, rate in shapes]
    i = next(j for j in range(len(shapes)) if cost[j] <= min(cost) * (1 + 1e-12))
    return shapes[i][:2]


def test_gemm_splitk_rule(lib):
    """K slices of gemm_splitk_*: only when the tiles leave CUs idle, at
    least 10 K tiles of 64 per slice, no empty slice, never on skinny shapes,
    and only when the K loop gets at least 12 + splits·M·N / 2^18 K tiles
    shorter."""
    want = {
        (1024, 1024, 4096): 4,     # 64 tiles of 128x128; 16 K tiles per slice
        (1024, 1024, 14336): 4,
        (512, 4096, 8192): 2,      # 128 tiles
        (512, 4096, 4096): 2,      # saves 32 K tiles, costs 12 + 16
        (1024, 1024, 2048): 1,     # 3 slices would save 21 K tiles, cost 12 + 12
        (300, 260, 4104): 6,       # 9 tiles; 65 K tiles -> slices of 11
        (128, 128, 14336): 21,     # one tile; 224 K tiles -> 22 slices of 11 -> 21 non-empty
        (128, 4096, 14336): 8,     # 32 tiles: 8 slices fill the CUs
        (2048, 1024, 2048): 1,     # 128 tiles; 2 slices would save 16 K tiles, cost 12 + 16
        (1024, 1024, 1024): 1,     # 16 K tiles: fewer than 2 x 10
        (4096, 4096, 4096): 1,     # 256 tiles already
        (8192, 1024, 8192): 1,     # 256 tiles of 256x128
        (16, 4096, 4096): 1,       # skinny kernel
        (4096, 1, 4096): 1,        # GEMV
    }
    for (M, N, K), splits in want.items():
        assert gt.splitk_splits(M, N, K, 256) == splits, (M, N, K)
        assert gt.splitk_workspace_bytes(M, N, K, 256) == (splits * M * N * 4 if splits > 1 else 0)
    # the documented formula, evaluated independently
    for M in (17, 100, 300, 777, 1024, 2049):
        for N in (17, 129, 1000, 3000):
            for K in (8, 448, 512, 1032, 1280, 4104, 14336):
                for cus in (80, 256):
                    bm, bn = _splitk_tile(M, N, cus)
                    T = -(-M // bm) * -(-N // bn)
                    kt = -(-K // 64)
                    s = 1
                    if T < cus and kt >= 2 * SPLITK_MIN_TILES:
                        s = min(cus // T, kt // SPLITK_MIN_TILES)
                        if s >= 2:
                            per = -(-kt // s)
                            s = -(-kt // per)
                            if kt * (s - 1) / s < SPLITK_MIN_SAVED + s * M * N / SPLITK_OUTPUTS_PER_TILE:
                                s = 1
                        else:
                            s = 1
                    assert gt.splitk_splits(M, N, K, cus) == s, (M, N, K, cus)
    assert gt.splitk_splits(0, 4, 8, 256) == 1 and gt.splitk_workspace_bytes(4, 4, 0, 256) == 0


def test_gemm_splitk_skinny_rule(lib):
    """K slices on the skinny kernel (2..16 rows on a side): K tiles of 512,
    at least 2 per slice, only while the blocks of 16 large-side rows leave
    CUs idle and KT >= 8 + 64·blocks/#CUs; one row on a side never splits."""
    want = {
        (8, 1024, 14336): 4,     # 64 blocks, 28 K tiles >= 8 + 16
        (8, 1024, 8192): 1,      # 16 K tiles < 24
        (8, 256, 14336): 14,     # 16 blocks; 28 K tiles -> 14 slices of 2
        (16, 64, 8192): 8,       # 4 blocks; 16 K tiles -> 8 slices of 2
        (8, 64, 4096): 1,        # 8 K tiles < 9
        (8, 2048, 14336): 1,     # 128 blocks: 28 < 8 + 32
        (8, 4096, 14336): 1,     # 256 blocks fill the CUs
        (1000, 5, 14336): 4,     # N <= 16: the same rule on the 1000 rows of A
        (1, 1024, 14336): 1,     # the GEMV
        (1024, 1, 14336): 1,
    }
    for (M, N, K), splits in want.items():
        assert gt.splitk_splits(M, N, K, 256) == splits, (M, N, K)
        assert gt.splitk_workspace_bytes(M, N, K, 256) == (splits * M * N * 4 if splits > 1 else 0)
    for S in (2, 5, 16):
        for R in (17, 100, 300, 777, 1024, 2049, 5000):
            for K in (8, 1032, 2048, 4104, 8192, 14336, 65536):
                for cus in (80, 256):
                    blocks = -(-R // 16)
                    kt = -(-K // 512)
                    s = 1
                    if blocks < cus and kt >= 4 and kt * cus >= 8 * cus + 64 * blocks:
                        s = min(cus // blocks, kt // 2)
                        if s >= 2:
                            per = -(-kt // s)
                            s = -(-kt // per)
                        else:
                            s = 1
                    assert gt.splitk_splits(S, R, K, cus) == s, (S, R, K, cus)
                    assert gt.splitk_splits(R, S, K, cus) == s, (R, S, K, cus)


def test_gemm_splitk_argument_validation(lib):
    for fn in (lib.gemm_splitk_f16, lib.gemm_splitk_bf16):
        assert fn(FAKE, FAKE, FAKE, 4, 4, 8, FAKE, -1, None) == INVALID  # negative workspace size
        assert fn(FAKE, FAKE, FAKE, -1, 4, 8, FAKE, 0, None) == INVALID
        assert fn(FAKE, FAKE, FAKE, 4, 4, 12, FAKE, 0, None) == UNSUPPORTED
        assert fn(None, None, None, 0, 4, 8, None, 0, None) == OK


def test_gemm_splitk_noalloc_argument_validation(lib):
    """The non-allocating split-K entry point checks its arguments like
    gemm_splitk_f16, before any HIP call."""
    fn = lib.gemm_splitk_f16_noalloc
    assert fn(FAKE, FAKE, FAKE, -1, 4, 8, None) == INVALID
    assert fn(FAKE, FAKE, None, 4, 4, 8, None) == INVALID
    assert fn(FAKE, FAKE, FAKE, 4, 4, 12, None) == UNSUPPORTED
    assert fn(FAKE + 8, FAKE, FAKE, 4, 4, 8, None) == UNSUPPORTED
    assert fn(None, None, None, 0, 4, 8, None) == OK
    assert "16 MiB" in gt.status_string(5)


NOALLOC_SCRATCH_BYTES = 16 << 20


def test_noalloc_scratch_covers_every_split_on_256_cus():
    """Split-K shapes take 128x128 tiles and tiles x splits <= #CUs, so on
    256 compute units no shape needs more than the 16 MiB static scratch of
    gemm_splitk_f16_noalloc; a larger part can (hence its size check)."""
    sizes = [1, 2, 15, 16, 17, 33, 64, 100, 128, 129, 255, 256, 300, 384, 512, 640, 768, 1000, 1024, 1280, 1536,
             2000, 2048, 3000, 4096, 8192]
    worst = 0
    for M in sizes:
        for N in sizes:
            for K in (1024, 4104, 14336, 65536, 1 << 20):
                worst = max(worst, gt.splitk_workspace_bytes(M, N, K, 256))
    assert 0 < worst <= NOALLOC_SCRATCH_BYTES
    assert gt.splitk_workspace_bytes(1024, 1024, 14336, 512) > NOALLOC_SCRATCH_BYTES


def test_measurement_formulas_match_table1():
    rows = {}
    for line in open(os.path.join(GOLDEN, "gemv_table1.txt")):
        if line.strip() and not line.startswith("#"):
            parts = line.split()
            rows[parts[0]] = [int(p) for p in parts[1:]]
    N, K = 4096, 14336
    el = metrics.gemv_elements(N, K)
    for name in ("W", "x", "y", "total"):
        assert el[name] == rows[name][0], name
        assert el[name] * metrics.FP16_BYTES == rows[name][1], name
    assert metrics.gemv_bytes(N, K) == rows["total"][1]
    assert metrics.gemv_flops(N, K) == rows["flops"][0]
    assert metrics.gemm_flops(4096, 4096, 4096) == 137438953472


def test_gemv_grid_gives_every_cu_a_workgroup(lib):
    """gemv_f16 splits K over the waves of a workgroup when N alone would
    leave compute units idle (16, 8, 4, 2 rows per workgroup, then 1), and
    always takes 2 rows per workgroup (K split 8 ways) for K >= 8192 while
    that gives every CU a workgroup."""
    K = 4096
    assert gt.gemv_grid(4096, K, 256) == 256  # 16 rows per workgroup, no split
    assert gt.gemv_grid(4097, K, 256) == 257
    assert gt.gemv_grid(8192, K, 256) == 512
    assert gt.gemv_grid(4095, K, 256) == 512  # 8 rows per workgroup
    assert gt.gemv_grid(2048, K, 256) == 256
    assert gt.gemv_grid(1024, K, 256) == 256  # 4 rows
    assert gt.gemv_grid(1031, K, 256) == 258
    assert gt.gemv_grid(512, K, 256) == 256  # 2 rows
    assert gt.gemv_grid(511, K, 256) == 511  # 1 row
    assert gt.gemv_grid(1, K, 256) == 1
    assert gt.gemv_grid(0, K, 256) == 0
    assert gt.gemv_grid(5, K, 0) == 0
    assert gt.gemv_grid(5, -8, 256) == 0
    # long rows: 2 rows per workgroup from N = 2 * CUs up
    assert gt.gemv_grid(4096, 8184, 256) == 256
    assert gt.gemv_grid(4096, 8192, 256) == 2048
    assert gt.gemv_grid(4096, 14336, 256) == 2048
    assert gt.gemv_grid(512, 14336, 256) == 256
    assert gt.gemv_grid(511, 14336, 256) == 511
    for K in (0, 8, 4096, 8184, 8192, 14336, 65536):
        for N in list(range(1, 70)) + [255, 256, 257, 1000, 3000, 4096, 10000, 14336]:
            for cus in (1, 8, 80, 256, 304):
                g = gt.gemv_grid(N, K, cus)
                assert g >= 1
                if N >= 2 * cus:
                    assert g >= cus  # every CU gets a workgroup
                # the documented rule: 2 rows per workgroup when K >= 8192
                # and N >= 2 * cus; else the largest of 16, 8, 4, 2 rows per
                # workgroup with N >= rows * cus, else 1
                if K >= 8192 and N >= 2 * cus:
                    rows = 2
                else:
                    rows = next((r for r in (16, 8, 4, 2) if N >= r * cus), 1)
                assert g == -(-N // rows)
