"""Pins for the oracle's MXFP4 operand dequantisation and FP4 GEMM.

What fixes the answer here (never the oracle's own formula):
* the quant-dequant output, already pinned by exact-rational brute force
  (tests/test_oracle_mxfp4.py): dequantising its codes and scales must give
  it back bit for bit;
* the page's printed codebook (tests/golden/mxfp4_numeric_model.txt) for the
  sixteen nibbles;
* numpy's fp64 matrix product of those quant-dequant outputs for the GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_mxfp4 import golden


def pack_nibbles(nibs: np.ndarray) -> np.ndarray:
    """[rows][2n] nibbles -> [rows][n] bytes, element 2j in the low nibble."""
    nibs = nibs.astype(np.uint8)
    return (nibs[:, 0::2] | (nibs[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("shape,sf", [((3, 17), 6.0), ((4, 45), 6.0), ((6, 100), 5.0), ((2, 256), 0.75),
                                      ((5, 64), 12.0)])
def test_dequant_reproduces_qdq_output(shape, sf):
    g = torch.Generator().manual_seed(shape[1])
    x = (torch.randn(shape, generator=g) * torch.exp2(torch.randint(-25, 25, (shape[0], 1), generator=g).float())).numpy()
    y, codes, scales, _ = oracle.mxfp4_qdq_ex(x, sf)
    d = oracle.mxfp4_dequant(codes, scales, shape[1])
    assert np.array_equal(d, y.astype(np.float64))
    assert np.array_equal(np.signbit(d), np.signbit(y))


def test_dequant_of_every_nibble_is_the_page_codebook():
    cb = [float(v) for v in golden()["codebook"]]
    nibs = np.tile(np.arange(16), 2)[None]                 # one row of 32 elements
    for s in (97, 126, 127, 128, 200):
        d = oracle.mxfp4_dequant(pack_nibbles(nibs), np.array([[s]], np.uint8), 32)[0]
        scale = 2.0 ** (s - 127)
        assert list(np.abs(d[:8]) / scale) == cb           # nibbles 0..7: the codebook, ascending
        assert list(np.abs(d[8:16]) / scale) == cb         # nibbles 8..15: the same magnitudes ...
        assert np.all(np.signbit(d[8:16])) and not np.any(np.signbit(d[:8]))   # ... negated (incl. -0)
        assert np.array_equal(d[16:], d[:16])


def test_gemm_fp4_equals_matmul_of_qdq_outputs():
    g = torch.Generator().manual_seed(3)
    M, N, K = 5, 7, 160
    xa = (torch.randn(M, K, generator=g) * torch.exp2(torch.randint(-8, 8, (M, 1), generator=g).float())).numpy()
    xb = (torch.randn(N, K, generator=g) * torch.exp2(torch.randint(-8, 8, (N, 1), generator=g).float())).numpy()
    ya, ca, sa, _ = oracle.mxfp4_qdq_ex(xa, 6.0)
    yb, cb, sb, _ = oracle.mxfp4_qdq_ex(xb, 6.0)
    C, Cabs = oracle.gemm_fp4(ca, sa, cb, sb)
    ref = ya.astype(np.float64) @ yb.astype(np.float64).T
    refabs = np.abs(ya.astype(np.float64)) @ np.abs(yb.astype(np.float64)).T
    assert np.all(np.abs(C - ref) <= 1e-12 * refabs)
    assert np.allclose(Cabs, refabs, rtol=1e-12, atol=0)
    # transposing the operands transposes the product
    Ct, _ = oracle.gemm_fp4(cb, sb, ca, sa)
    assert np.array_equal(Ct, C.T)


def test_gemm_fp4_sampled_equals_full():
    g = torch.Generator().manual_seed(4)
    xa, xb = torch.randn(9, 96, generator=g).numpy(), torch.randn(11, 96, generator=g).numpy()
    _, ca, sa, _ = oracle.mxfp4_qdq_ex(xa, 6.0)
    _, cb, sb, _ = oracle.mxfp4_qdq_ex(xb, 6.0)
    C, Cabs = oracle.gemm_fp4(ca, sa, cb, sb)
    mi = np.array([0, 8, 3, 5, 8]); ni = np.array([0, 10, 7, 2, 0])
    Cs, Cas = oracle.gemm_fp4_sampled(ca, sa, cb, sb, mi, ni)
    assert np.allclose(Cs, C[mi, ni], rtol=1e-13, atol=0) and np.allclose(Cas, Cabs[mi, ni], rtol=1e-13, atol=0)


def test_grouped_token_axis_fp4_operand():
    """The grouped token-axis MXFP4 operand: one group is the QDQ of the
    transpose; groups restart their blocks (a group's codes do not depend on
    its neighbours' tokens); tails and unused positions are zero codes; the
    dequantised operand reproduces the QDQ of each group's transposed rows."""
    rng = np.random.default_rng(5)
    T, C = 90, 40
    x = (rng.standard_normal((T, C)) * np.exp2(rng.integers(-6, 6, (T, 1)))).astype(np.float32)
    ge = np.array([0, 33, 33, 70, 90], np.int32)
    ldq = 224
    codes, scales = oracle.mxfp4_quant_grouped_colT(x, ge, ldq)
    # one group: the QDQ of the transpose
    c1, s1 = oracle.mxfp4_quant_grouped_colT(x, np.array([T], np.int32), 96)
    _, cr, sr, _ = oracle.mxfp4_qdq_ex(np.ascontiguousarray(x.T))
    assert np.array_equal(c1, cr) and np.array_equal(s1, sr)
    # sizes 0, 33, 0, 37, 20: padded positions [0, 64), [64, 128), [128, 160)
    # group 3 (rows 33..70) alone gives the same bytes as inside the grouped copy
    P2 = 64
    cg, sg = oracle.mxfp4_quant_grouped_colT(np.ascontiguousarray(x[33:70]), np.array([37], np.int32), 64)
    assert np.array_equal(codes[:, P2 // 2:(P2 + 64) // 2], cg[:, :32])
    assert np.array_equal(scales[:, P2 // 32:(P2 + 64) // 32], sg[:, :2])
    # padding: group 1 (33 tokens) occupies 64 positions, its last 31 are zero codes
    assert not codes[:, 33 // 2 + 1:64 // 2].any() and not (codes[:, 16] >> 4).any()
    assert not codes[:, 160 // 2:].any() and not scales[:, 160 // 32:].any()
    # dequantised operand = QDQ values of each group's transposed rows
    deq = oracle.mxfp4_dequant(codes, scales, ldq)
    start, P = 0, 0
    for e in ge.tolist():
        m = e - start
        if m:
            y, _, _, _ = oracle.mxfp4_qdq_ex(np.ascontiguousarray(x[start:e].T))
            assert np.array_equal(deq[:, P:P + m], y.astype(np.float64))
        P += (m + 31) // 32 * 32
        start = e
