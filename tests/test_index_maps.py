"""Host replicas of the MXFP8 quantisers' workgroup-to-work mappings
(quant_mxfp8.hip).  Row quantiser: unit u covers rows 32 j + (u % per_group)
* rps + i of 128-row group u / per_group, and workgroup b runs the unit that
puts every workgroup of one group on the XCD b % 8.  Ungrouped tile
quantiser: workgroup b runs the tile that gives each XCD eight consecutive
tiles.  Each mapping must be a permutation, so every row or tile is
quantised exactly once, for every size, full runs or not."""
import pytest


def row_unit(b, n_units, per_group):
    span = 8 * per_group
    full = n_units // span * span
    if b < full:
        r = b % span
        return b - r + (r & 7) * per_group + (r >> 3)
    return b


def launch_shape(R, C):
    """tpr_log2, per_group and units as the launcher and kernel derive them."""
    cpr = (C + 31) // 32 * 4
    tpr_log2 = 3
    while (1 << tpr_log2) < cpr and tpr_log2 < 8:
        tpr_log2 += 1
    per_group = 32 >> (8 - tpr_log2)
    return per_group, (R + 127) // 128 * per_group


@pytest.mark.parametrize("R", [1, 127, 128, 1000, 8 * 128, 8 * 128 + 1, 131072])
@pytest.mark.parametrize("C", [1, 32, 100, 512, 1024, 4096, 7168])
def test_row_units_are_a_permutation(R, C):
    per_group, n_units = launch_shape(R, C)
    units = [row_unit(b, n_units, per_group) for b in range(n_units)]
    assert sorted(units) == list(range(n_units))
    span = 8 * per_group
    full = n_units // span * span
    # within full runs, a group's workgroups share one XCD
    for b in range(full):
        assert (units[b] // per_group) % 8 == b % 8


def tile_of(b, grid):
    full = grid // 64 * 64
    if b < full:
        r = b & 63
        return b - r + (r & 7) * 8 + (r >> 3)
    return b


@pytest.mark.parametrize("grid", [1, 63, 64, 65, 1000, 4096, 14680064 // 256])
def test_tile_order_is_a_permutation(grid):
    tiles = [tile_of(b, grid) for b in range(grid)]
    assert sorted(tiles) == list(range(grid))
    for b in range(grid // 64 * 64):   # eight consecutive tiles per XCD
        assert (tiles[b] // 8) % 8 == b % 8



FP4_UNITS = 2   # 1024-element row pieces per workgroup of the MXFP4 operand row quantiser


@pytest.mark.parametrize("rows", [1, 3, 127, 128, 129, 1029, 18432])
@pytest.mark.parametrize("L", [1024, 3072, 4096, 7168])
def test_fp4_operand_rows_cover_every_piece_once(rows, L):
    """MXFP4 operand row quantiser (qdq_mxfp4.hip): workgroup w takes pieces
    2w and 2w + 1 (those below rows * L / 1024); the first piece's row and
    place come from one division and the next piece follows, wrapping to the
    next row."""
    upr = L // 1024
    n_units = rows * upr
    n_wg = (n_units + FP4_UNITS - 1) // FP4_UNITS
    seen = []
    for w in range(n_wg):
        row, seg = divmod(w * FP4_UNITS, upr)
        for k in range(FP4_UNITS):
            u = w * FP4_UNITS + k
            if u < n_units:
                assert u == row * upr + seg and 0 <= row < rows   # element 1024 u = row * L + 1024 seg
                seen.append((row, seg))
            seg += 1
            if seg == upr:
                seg, row = 0, row + 1
    assert seen == [(r, g) for r in range(rows) for g in range(upr)]


FP4_GROUP_COL_TILES = 4   # column tiles of one row tile walked by a workgroup of the MXFP4 grouped quantiser
FP8_GROUP_COL_TILES = 4   # the same for the MXFP8 grouped token-axis copy (quant_mxfp8.hip)


@pytest.mark.parametrize("C", [1, 31, 32, 33, 96, 128, 129, 200, 511, 513, 4096, 7168])
@pytest.mark.parametrize("n_row_tiles", [1, 3, 516])
@pytest.mark.parametrize("col_tile, walk", [(32, FP4_GROUP_COL_TILES), (128, FP8_GROUP_COL_TILES)])
def test_grouped_column_walk_covers_every_tile_once(C, n_row_tiles, col_tile, walk):
    """Grouped token-axis quantisers (MXFP4: 32-column tiles, qdq_mxfp4.hip;
    MXFP8: 128-column tiles, quant_mxfp8.hip): workgroup b takes row tile
    b / n_col_groups and column tiles [walk (b % n_col_groups), + walk) cut at
    n_col_tiles; the launcher sizes the grid n_row_tiles x n_col_groups."""
    n_col_tiles = (C + col_tile - 1) // col_tile
    n_col_groups = (n_col_tiles + walk - 1) // walk
    seen = []
    for b in range(n_row_tiles * n_col_groups):
        rt = b // n_col_groups
        ct_begin = (b - rt * n_col_groups) * walk
        ct_end = min(ct_begin + walk, n_col_tiles)
        assert 0 <= rt < n_row_tiles and ct_begin < ct_end
        seen += [(rt, ct) for ct in range(ct_begin, ct_end)]
    assert seen == [(r, c) for r in range(n_row_tiles) for c in range(n_col_tiles)]


def test_replica_constants_match_the_kernel_source():
    """The replicas above use the kernels' own constants."""
    import re
    from pathlib import Path
    src = (Path(__file__).resolve().parents[1] / "moe_grouped_gemm_mxq_amd" / "csrc" / "qdq_mxfp4.hip").read_text()
    assert int(re.search(r"constexpr int kOpUnits = (\d+);", src).group(1)) == FP4_UNITS
    assert int(re.search(r"constexpr int kGrpColTiles = (\d+);", src).group(1)) == FP4_GROUP_COL_TILES
    src8 = (Path(__file__).resolve().parents[1] / "moe_grouped_gemm_mxq_amd" / "csrc" / "quant_mxfp8.hip").read_text()
    assert int(re.search(r"constexpr int kGrpWalk = (\d+);", src8).group(1)) == FP8_GROUP_COL_TILES
    assert re.search(r"constexpr int kTR = 128, kTC = (\d+),", src8).group(1) == "128"
