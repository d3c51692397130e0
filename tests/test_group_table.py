"""Host replica of the device group-table arithmetic (mxq_groups.h) and of
the index computations its users derive from it, run on group_end arrays
that break the precondition (not non-decreasing, negative, past the row
count, INT32_MAX).  The device code must keep every access in bounds for
them; this checks the arithmetic on the CPU, where an overflow or an
out-of-range index is an assertion, before any GPU runs such an array.

The replica follows the kernels step by step:
  * build_block_starts: ends clamped into [0, R], per-group unit counts
    ceil((size + start % align) / unit) in 64 bits, prefix sums saturated at
    INT32_MAX;
  * the grouped quantisers (MXFP8 tiles of 128 padded positions, MXFP4 of
    256): padded block pb -> group g (largest g with bstart[g] <= pb), source
    rows [gstart + off, + valid);
  * the ragged-M GEMM: m-tile -> (group, first row m0, rows), tile count cut
    at the launcher's bound tiles_m + 2G;
  * the ragged-K GEMM: expert g's reduction range [k_begin, k_end) in [0, K],
    read from the 128-byte line at or below k_begin (the head zeroed).
"""
import numpy as np
import pytest

INT32_MAX = 2 ** 31 - 1


def group_span(ge, g, R):
    e = int(ge[g])
    b = int(ge[g - 1]) if g else 0
    e = min(max(e, 0), R)
    b = min(max(b, 0), R)
    return b, (e - b if e > b else 0)


def build_block_starts(ge, R, unit, align=1):
    G = len(ge)
    start, size, nb = [], [], []
    for g in range(G):
        b, m = group_span(ge, g, R)
        start.append(b)
        size.append(m)
        nb.append((m + b % align + unit - 1) // unit if m > 0 else 0)
    bstart, run = [], 0
    for g in range(G):
        bstart.append(min(run, INT32_MAX))
        run += nb[g]
    bstart.append(min(run, INT32_MAX))
    assert all(0 <= v <= INT32_MAX for v in bstart)
    return start, size, bstart, nb


def find_group(bstart, G, u):
    lo, hi = 0, G - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if bstart[mid] <= u:
            lo = mid
        else:
            hi = mid - 1
    return lo


ARRAYS = [
    [INT32_MAX, 0, 100],
    [0, INT32_MAX, 7, INT32_MAX, 40],
    [-5, 70, 30, INT32_MAX],
    [INT32_MAX, 0] * 512,
    [INT32_MAX] * 1024,
    [-(2 ** 31)] * 7 + [5],
    list(np.random.default_rng(0).integers(-(2 ** 31), 2 ** 31, 1024)),
    list(np.random.default_rng(1).integers(0, 200, 300)),
]


def sample_units(total, n=4000, seed=0):
    if total <= n:
        return range(total)
    rng = np.random.default_rng(seed)
    return sorted(set(rng.integers(0, total, n).tolist()) | {0, total - 1})


@pytest.mark.parametrize("ends", ARRAYS)
@pytest.mark.parametrize("T", [1, 96, 5000])
@pytest.mark.parametrize("tile_rows", [128, 256])  # MXFP8 tile quantiser / grouped MXFP4 quantiser
def test_grouped_quantiser_reads_inside_the_input(ends, T, tile_rows):
    G = len(ends)
    ldq = (((T + 31 * G + 255) // 256) | 1) * 256  # mxq_grouped_cols_max: an odd multiple of 256
    start, size, bstart, nb = build_block_starts(ends, T, 32)
    assert all(bstart[g] <= bstart[g + 1] <= bstart[g] + nb[g] for g in range(G))
    # tiles of tile_rows padded positions over T + 31 G
    launched_blocks = (T + 31 * G + tile_rows - 1) // tile_rows * (tile_rows // 32)
    for pb in sample_units(min(bstart[G], launched_blocks)):
        if (pb + 1) * 32 > ldq:
            continue                                    # the kernel drops such blocks
        g = find_group(bstart, G, pb)
        assert bstart[g] <= pb < bstart[g + 1]
        off = (pb - bstart[g]) * 32
        src, valid = start[g] + off, min(32, size[g] - off)
        assert valid >= 1 and src >= 0 and src + valid <= T, (g, pb, off, src, valid)


@pytest.mark.parametrize("ends", ARRAYS)
@pytest.mark.parametrize("M", [1, 96, 1000])
def test_ragged_m_tiles_stay_inside_the_rows(ends, M):
    G, BM, tiles_n = len(ends), 256, 3
    tiles_m = (M + BM - 1) // BM
    start, size, bstart, nb = build_block_starts(ends, M, BM, align=128)
    n_tiles = min(bstart[G], tiles_m + 2 * G) * tiles_n
    assert n_tiles < 2 ** 31
    for mt in sample_units(n_tiles // tiles_n):
        g = find_group(bstart, G, mt)
        local = mt - bstart[g]
        assert 0 <= local < nb[g]
        m_al = start[g] & ~127
        m0 = m_al + local * BM
        rows_a = min(BM, start[g] + size[g] - m0)
        rows_load = min(BM, M - m0)
        row_lo = start[g] - m_al if local == 0 else 0
        assert 0 <= m0 < M and 1 <= rows_load and rows_a <= rows_load, (g, mt, m0, rows_a, rows_load)
        assert 0 <= row_lo < BM


@pytest.mark.parametrize("ends", ARRAYS)
@pytest.mark.parametrize("K", [32, 192, 4096])
def test_ragged_k_ranges_stay_inside_the_reduction(ends, K):
    G = len(ends)
    start, size, kb, nb = build_block_starts(ends, K, 32)
    n_long = sum(1 for m in size if m > 1024)
    assert 0 <= n_long <= G
    for g in range(G):
        k_begin = min(kb[g] * 32, K)
        k_end = min(kb[g + 1] * 32, K)
        assert 0 <= k_begin <= K and 0 <= k_end <= K
        klen = k_end - k_begin if k_end > k_begin else 0
        assert k_begin + klen <= K
        # the plain launch starts at the 128-byte line at or below k_begin (128
        # E4M3 or 256 E2M1 tokens) and zeroes the head chunks (16 or 32 tokens)
        for stage_elems, chunk_elems in ((128, 16), (256, 32)):
            if klen > 0:
                al = k_begin // stage_elems * stage_elems
                head_chunks = (k_begin - al) // chunk_elems
                assert 0 <= al <= k_begin and (k_begin - al) % chunk_elems == 0
                assert 0 <= head_chunks < stage_elems // chunk_elems
                assert al + (klen + k_begin - al) == k_end <= K


def test_valid_arrays_are_unchanged():
    """For a valid (non-decreasing, <= R) array the clamps change nothing:
    block starts are the plain prefix sums of ceil(size / unit)."""
    rng = np.random.default_rng(3)
    sizes = rng.integers(0, 700, 100)
    ends = np.cumsum(sizes).tolist()
    _, size, bstart, _ = build_block_starts(ends, int(ends[-1]), 32)
    assert size == sizes.tolist()
    assert bstart == np.concatenate([[0], np.cumsum((sizes + 31) // 32)]).tolist()
