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
