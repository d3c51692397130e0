"""The MXFP4 kernels find the E2M1 codebook index of yabs = |x| * 2^-e from a
table keyed by the exponent and top two mantissa bits of yabs (mxq_device.h,
kFp4IndexTable).  Check that table, read from the header, against the
definition: the number of codebook midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5
that yabs reaches (ties to the larger magnitude, AMCT FakeQuant article,
section 2), for every fp32 value of the binades where the index changes and
for samples of all the others."""
import os
import re

import numpy as np

HDR = os.path.join(os.path.dirname(__file__), "..", "moe_grouped_gemm_mxq_amd", "csrc", "mxq_device.h")
MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)


def table():
    m = re.search(r"kFp4IndexTable\s*=\s*(0x[0-9a-fA-F]+)ull", open(HDR).read())
    assert m, "kFp4IndexTable not found"
    return int(m.group(1), 16)


def index_from_table(u: np.ndarray, tab: int) -> np.ndarray:
    k = np.clip(u >> 21, 499, 519).astype(np.uint64) - 499
    return ((np.uint64(tab) >> (np.uint64(3) * k)) & np.uint64(7)).astype(np.int64)


def index_by_midpoints(u: np.ndarray) -> np.ndarray:
    y = u.view(np.float32)
    return (y[:, None] >= MIDPOINTS[None, :]).sum(axis=1)


def test_index_table_every_value_of_the_changing_binades():
    tab = table()
    for ef in range(122, 132):  # yabs in [2^-5, 2^5): every threshold and both clamps
        u = (np.uint32(ef) << np.uint32(23)) | np.arange(1 << 23, dtype=np.uint32)
        for part in np.array_split(u, 8):
            assert np.array_equal(index_from_table(part, tab), index_by_midpoints(part)), f"exponent field {ef}"


def test_index_table_elsewhere():
    tab = table()
    rng = np.random.default_rng(0)
    u = rng.integers(0, 0x7F800000, 4_000_000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, np.array([0, 1, 0x007FFFFF, 0x00800000, 0x7F7FFFFF], np.uint32)])
    assert np.array_equal(index_from_table(u, tab), index_by_midpoints(u))
