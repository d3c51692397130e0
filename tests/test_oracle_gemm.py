"""Pins for the oracle's block-scaled dense and grouped GEMMs.

What fixes the answer (never the oracle's own formula):
* numpy's float64 matmul of operands dequantised through PyTorch's
  ``float8_e4m3fn`` and 2^(byte-127) (a textbook routine on an independent
  decode);
* exact cases: one-hot code rows select single products exactly;
* reductions: a ragged-M grouped GEMM is a dense GEMM per group; a ragged-K
  one is a dense GEMM over each group's padded column range; an empty group
  gives exact zeros; sampled entry points equal the full ones.
"""
import numpy as np
import pytest
import torch

import oracle


def deq_torch(q, s):
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v * np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)


def rand_operand(rng, R, K, lo=100, hi=150):
    q = rng.integers(0, 256, (R, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x11               # no NaN codes
    s = rng.integers(lo, hi, (R, K // 32), dtype=np.uint8)
    return q, s


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (17, 9, 96), (64, 48, 512)])
def test_gemm_equals_numpy_matmul_of_dequantised(M, N, K):
    rng = np.random.default_rng(M + N + K)
    A, sA = rand_operand(rng, M, K)
    B, sB = rand_operand(rng, N, K)
    C, Cabs = oracle.gemm(A, sA, B, sB)
    a, b = deq_torch(A, sA), deq_torch(B, sB)
    ref = a @ b.T
    refabs = np.abs(a) @ np.abs(b).T
    assert np.allclose(C, ref, rtol=0, atol=1e-13 * refabs.max())
    assert np.allclose(Cabs, refabs, rtol=1e-13, atol=0)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (33, 70, 160), (96, 40, 1024)])
def test_gemm_dequantised_equals_gemm(M, N, K):
    """The full-size checks' BLAS route (dequantise, then an fp64 matrix
    product) gives the plain loops' sums up to fp64 rounding order."""
    rng = np.random.default_rng(7 * M + N + K)
    A, sA = rand_operand(rng, M, K, lo=90, hi=160)
    B, sB = rand_operand(rng, N, K, lo=90, hi=160)
    C, Cabs = oracle.gemm(A, sA, B, sB)
    C2, Cabs2 = oracle.gemm_dequantised(oracle.mxfp8_dequant(A, sA), oracle.mxfp8_dequant(B, sB))
    assert np.all(np.abs(C2 - C) <= 1e-13 * Cabs)
    assert np.all(np.abs(Cabs2 - Cabs) <= 1e-13 * Cabs)


def test_gemm_one_hot_rows_select_products_exactly():
    K = 128
    A = np.zeros((4, K), np.uint8)
    sA = np.full((4, K // 32), 127, np.uint8)
    for m in range(4):
        A[m, 37 * m + 5] = 0x38                    # 1.0
    sA[2, :] = 130                                 # scale 2^3 on row 2
    rng = np.random.default_rng(1)
    B, sB = rand_operand(rng, 6, K)
    C, _ = oracle.gemm(A, sA, B, sB)
    b = deq_torch(B, sB)
    for m in range(4):
        k = 37 * m + 5
        assert np.array_equal(C[m], b[:, k] * (8.0 if m == 2 else 1.0))


def test_gemm_sampled_equals_full():
    rng = np.random.default_rng(2)
    A, sA = rand_operand(rng, 33, 64)
    B, sB = rand_operand(rng, 20, 64)
    C, Cabs = oracle.gemm(A, sA, B, sB)
    mi = rng.integers(0, 33, 200)
    ni = rng.integers(0, 20, 200)
    c, cabs = oracle.gemm_sampled(A, sA, B, sB, mi, ni)
    assert np.array_equal(c, C[mi, ni]) and np.array_equal(cabs, Cabs[mi, ni])


@pytest.mark.parametrize("sizes", [[5, 0, 33, 1, 25], [0, 0, 64], [64]])
def test_ragged_m_is_dense_per_group(sizes):
    rng = np.random.default_rng(len(sizes))
    T, K, N, G = sum(sizes), 96, 24, len(sizes)
    A, sA = rand_operand(rng, T + 3, K)             # 3 trailing rows in no group
    Bq = np.stack([rand_operand(rng, N, K)[0] for _ in range(G)])
    Bs = np.stack([rand_operand(rng, N, K)[1] for _ in range(G)])
    ge = np.cumsum(sizes).astype(np.int32)
    C, Cabs = oracle.grouped_gemm_ragged_m(A, sA, Bq, Bs, ge)
    start = 0
    for g, m in enumerate(sizes):
        if m:
            Cg, Cgabs = oracle.gemm(A[start:start + m], sA[start:start + m], Bq[g], Bs[g])
            assert np.array_equal(C[start:start + m], Cg) and np.array_equal(Cabs[start:start + m], Cgabs)
        start += m
    assert np.all(C[T:] == 0)
    mi = rng.integers(0, T, 50)
    ni = rng.integers(0, N, 50)
    c, cabs = oracle.grouped_gemm_ragged_m_sampled(A, sA, Bq, Bs, ge, mi, ni)
    assert np.array_equal(c, C[mi, ni]) and np.array_equal(cabs, Cabs[mi, ni])


@pytest.mark.parametrize("sizes", [[5, 0, 33, 1, 40], [0, 64, 0], [32]])
def test_ragged_k_is_dense_per_group_and_empty_is_zero(sizes):
    rng = np.random.default_rng(10 + len(sizes))
    M, N, G = 20, 12, len(sizes)
    ge = np.cumsum(sizes).astype(np.int32)
    ldk = oracle.grouped_cols(ge) + 32
    A, sA = rand_operand(rng, M, ldk)
    B, sB = rand_operand(rng, N, ldk)
    C, Cabs = oracle.grouped_gemm_ragged_k(A, sA, B, sB, ge)
    P = 0
    for g, m in enumerate(sizes):
        w = oracle.ceil32(m)
        if w:
            Cg, Cgabs = oracle.gemm(np.ascontiguousarray(A[:, P:P + w]), np.ascontiguousarray(sA[:, P // 32:(P + w) // 32]),
                                    np.ascontiguousarray(B[:, P:P + w]), np.ascontiguousarray(sB[:, P // 32:(P + w) // 32]))
            assert np.array_equal(C[g], Cg) and np.array_equal(Cabs[g], Cgabs)
        else:
            assert np.array_equal(C[g], np.zeros((M, N))) and np.all(Cabs[g] == 0)
        P += w
    gi = rng.integers(0, G, 60).astype(np.int32)
    mi = rng.integers(0, M, 60)
    ni = rng.integers(0, N, 60)
    c, cabs = oracle.grouped_gemm_ragged_k_sampled(A, sA, B, sB, ge, gi, mi, ni)
    assert np.array_equal(c, C[gi, mi, ni]) and np.array_equal(cabs, Cabs[gi, mi, ni])


def test_end_to_end_linear_forward_small():
    """Quantise X along K (rows) and W along K (columns), multiply: the result
    equals numpy's matmul of the dequantised operands, and it approximates the
    unquantised product to within the format's relative precision."""
    from moe_grouped_gemm_mxq_amd.workloads import bf16_bits, linear_small
    X, W = linear_small()
    qa, sa = oracle.mxfp8_quant_row(bf16_bits(X))
    qb, sb = oracle.mxfp8_quant_colT(bf16_bits(W))
    C, Cabs = oracle.gemm(qa, sa, qb, sb)
    ref = deq_torch(qa, sa) @ deq_torch(qb, sb).T
    assert np.allclose(C, ref, rtol=0, atol=1e-12)
    exact = X.double().numpy() @ W.double().numpy()
    # each E4M3 element carries a relative error of at most 2^-4
    assert np.all(np.abs(C - exact) <= 2 * 2.0 ** -4 * Cabs + 1e-12)
