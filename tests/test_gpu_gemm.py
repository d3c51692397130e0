"""GPU parity of the dense block-scaled GEMM against the fp64 oracle:
|C_gpu - C_ref| <= 1e-5 * sum_k |a_k b_k| per element.  The oracle quantises
the seeded bf16 inputs itself and multiplies its own codes."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_gemm_close, bits, boundary_indices, host, mfma_group_bound, mxq, scale_rows,
                      scaled_randn, unpack_scales)
from moe_grouped_gemm_mxq_amd import workloads

pytestmark = pytest.mark.gpu


def gemm_case(M, N, K, seed):
    """X [M][K] row-quantised and W [K][N] column-quantised (the forward form)."""
    m = mxq()
    X = scaled_randn((M, K), seed, lo=-8, hi=8, zero_rows=min(1, M // 4))
    W = scaled_randn((K, N), seed + 1, lo=-8, hi=8, axis=1)
    qa = m.quantize(X.cuda(), 1)
    qb = m.quantize(W.cuda(), 2)
    C = m.gemm(qa["q_row"], qa["s_row"], qb["q_colT"], qb["s_colT"])
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_row(bits(X))
    B, sB = oracle.mxfp8_quant_colT(bits(W))
    Cr, Ca = oracle.gemm(A, sA, B, sB)
    return host(C), Cr, Ca, mfma_group_bound(A, sA, B, sB)


# (300, 300, 32) and (300, 300, 160): several tiles with one and two real
# K stages, the last one partial; tiles on odd (m-tile + n-tile) walk K one
# stage behind and start on that partial stage
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (16, 16, 128), (17, 33, 96), (256, 256, 512),
                                   (300, 260, 544), (513, 257, 1056), (64, 600, 4128),
                                   (300, 300, 32), (300, 300, 160)])
def test_gemm_shapes_with_tails(M, N, K):
    C, Cr, Ca, hw = gemm_case(M, N, K, seed=M + N + K)
    ratio = assert_gemm_close(C, Cr, Ca, f"gemm {M}x{N}x{K}", hw_bound=hw)
    print(f"gemm {M}x{N}x{K}: max err/sum|ab| = {ratio:.3e}")
    zero = Ca == 0
    assert np.all(C[zero] == 0.0)


def test_gemm_hardware_precision_model():
    """Values spread over 2^16 inside one K-block (W scaled per K-row) exceed
    what the FP8 MFMA's 8-product internal sums keep; the result still obeys
    the measured model |err| <= 1e-5*sum|ab| + 2^-10*sum_groups max|product|."""
    m = mxq()
    X = scaled_randn((96, 512), 21, lo=-8, hi=8)
    W = scaled_randn((512, 80), 22, lo=-8, hi=8, axis=0)
    qa, qb = m.quantize(X.cuda(), 1), m.quantize(W.cuda(), 2)
    C = host(m.gemm(qa["q_row"], qa["s_row"], qb["q_colT"], qb["s_colT"]))
    A, sA = oracle.mxfp8_quant_row(bits(X))
    B, sB = oracle.mxfp8_quant_colT(bits(W))
    Cr, Ca = oracle.gemm(A, sA, B, sB)
    err = np.abs(C - Cr)
    bound = 1e-5 * Ca + mfma_group_bound(A, sA, B, sB)
    assert np.all(err <= bound), float(np.max(err / bound))
    print(f"adversarial: max err/sum|ab| = {np.max(err / np.where(Ca > 0, Ca, 1)):.3e}, "
          f"max err/model bound = {np.max(err / bound):.3f}")


def test_gemm_ldc_wider_than_n():
    m = mxq()
    X = scaled_randn((70, 96), 3)
    W = scaled_randn((96, 50), 4, axis=1)
    qa, qb = m.quantize(X.cuda(), 1), m.quantize(W.cuda(), 2)
    Cbig = torch.full((70, 64), 7.0, device="cuda")
    m.mxq_gemm(qa["q_row"], qa["s_row"], qb["q_colT"], qb["s_colT"], Cbig)
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_row(bits(X))
    B, sB = oracle.mxfp8_quant_colT(bits(W))
    Cr, Ca = oracle.gemm(A, sA, B, sB)
    assert_gemm_close(host(Cbig)[:, :50], Cr, Ca, "ldc", hw_bound=mfma_group_bound(A, sA, B, sB))
    assert np.all(host(Cbig)[:, 50:] == 7.0)      # columns past N untouched


def test_gemm_is_deterministic():
    m = mxq()
    X = scaled_randn((512, 1024), 5)
    W = scaled_randn((1024, 384), 6, axis=1)
    qa, qb = m.quantize(X.cuda(), 1), m.quantize(W.cuda(), 2)
    c1 = m.gemm(qa["q_row"], qa["s_row"], qb["q_colT"], qb["s_colT"])
    c2 = m.gemm(qa["q_row"], qa["s_row"], qb["q_colT"], qb["s_colT"])
    assert torch.equal(c1, c2)


def test_linear_forward_small_end_to_end():
    """X bf16 [256x512], W bf16 [512x256], N(0,1) seed 0: quantise X by rows and W
    by columns (codes bit-exact), multiply (within tolerance)."""
    m = mxq()
    X, W = workloads.linear_small()
    qa, qb = m.quantize(X.cuda(), 1), m.quantize(W.cuda(), 2)
    C = m.gemm(qa["q_row"], qa["s_row"], qb["q_colT"], qb["s_colT"])
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_row(bits(X))
    B, sB = oracle.mxfp8_quant_colT(bits(W))
    assert np.array_equal(host(qa["q_row"]), A) and np.array_equal(unpack_scales(qa["s_row"], len(sA)), sA)
    assert np.array_equal(host(qb["q_colT"]), B) and np.array_equal(unpack_scales(qb["s_colT"], len(sB)), sB)
    Cr, Ca = oracle.gemm(A, sA, B, sB)
    ratio = assert_gemm_close(host(C), Cr, Ca, "linear 256x512x256", hw_bound=mfma_group_bound(A, sA, B, sB))
    print(f"linear 256x512x256: max err/sum|ab| = {ratio:.3e}")


def test_dense_fb_split_equals_dual():
    """fb-split quantises X by rows and W by columns in the forward and
    re-quantises X along M and W along N in the backward; every copy and the
    input / weight gradients equal the dual-axis schedule's bit for bit."""
    m = mxq()
    M, K, N = 300, 544, 260
    X = scaled_randn((M, K), 31, lo=-6, hi=6)
    W = scaled_randn((K, N), 32, lo=-6, hi=6, axis=1)
    dY = scaled_randn((M, N), 33, lo=-6, hi=6)
    Xd, Wd, dYd = X.cuda(), W.cuda(), dY.cuda()
    dual_x, dual_w = m.quantize(Xd, 3), m.quantize(Wd, 3)
    fb_x = {**m.quantize(Xd, 1), **m.quantize(Xd, 2)}   # forward rows, backward columns
    fb_w = {**m.quantize(Wd, 2), **m.quantize(Wd, 1)}
    # every copy equal (scales: the rows the operand has; padding rows are unspecified)
    for k in ("q_row", "q_colT"):
        assert torch.equal(dual_x[k], fb_x[k]) and torch.equal(dual_w[k], fb_w[k]), k
    for k, rx, rw in (("s_row", M, K), ("s_colT", K, N)):
        assert np.array_equal(unpack_scales(dual_x[k], rx), unpack_scales(fb_x[k], rx)), k
        assert np.array_equal(unpack_scales(dual_w[k], rw), unpack_scales(fb_w[k], rw)), k
    qy = m.quantize(dYd, 3)
    grads = []
    for qx, qw in ((dual_x, dual_w), (fb_x, fb_w)):
        dX = m.gemm(qy["q_row"], qy["s_row"], qw["q_row"], qw["s_row"])
        dW = m.gemm(qx["q_colT"], qx["s_colT"], qy["q_colT"], qy["s_colT"])
        grads.append((dX, dW))
    torch.cuda.synchronize()
    assert torch.equal(grads[0][0], grads[1][0]) and torch.equal(grads[0][1], grads[1][1])
    # and the gradients are right: dX = dY W^T against the oracle
    A, sA = oracle.mxfp8_quant_row(bits(dY))
    B, sB = oracle.mxfp8_quant_row(bits(W))
    Cr, Ca = oracle.gemm(A, sA, B, sB)
    assert_gemm_close(host(grads[1][0]), Cr, Ca, "fb-split dgrad", hw_bound=mfma_group_bound(A, sA, B, sB))


# ------------------------------------------------------------------ full size
@pytest.fixture(scope="module")
def dense_full():
    """Dense linear fwd / dgrad / wgrad at M=8192, K=7168, N=18432 with
    dual-axis quantisation of X, W and dY."""
    m = mxq()
    X, W, dY = workloads.dense_linear(device="cuda")
    qx, qw, qy = m.quantize(X, 3), m.quantize(W, 3), m.quantize(dY, 3)
    Y = m.gemm(qx["q_row"], qx["s_row"], qw["q_colT"], qw["s_colT"])       # [8192][18432]
    dX = m.gemm(qy["q_row"], qy["s_row"], qw["q_row"], qw["s_row"])        # [8192][7168]
    dW = m.gemm(qx["q_colT"], qx["s_colT"], qy["q_colT"], qy["s_colT"])    # [7168][18432]
    torch.cuda.synchronize()
    return dict(X=X, W=W, dY=dY, qx=qx, qw=qw, qy=qy, Y=Y, dX=dX, dW=dW)


def sample_rows(t: torch.Tensor, idx) -> np.ndarray:
    return bits(t[torch.as_tensor(idx, device=t.device)])


def sample_cols(t: torch.Tensor, idx) -> np.ndarray:
    return bits(t[:, torch.as_tensor(idx, device=t.device)].contiguous())


def test_dense_full_quantised_copies_sampled(dense_full):
    rng = np.random.default_rng(0)
    for name, src in (("qx", "X"), ("qw", "W"), ("qy", "dY")):
        x = dense_full[src]
        q = dense_full[name]
        R, C = x.shape
        rows = boundary_indices(R, 32, rng, 48)
        qr, sr = oracle.mxfp8_quant_row(sample_rows(x, rows))
        assert np.array_equal(host(q["q_row"][torch.as_tensor(rows, device="cuda")]), qr), name
        assert np.array_equal(scale_rows(q["s_row"], rows), sr), name
        cols = boundary_indices(C, 128, rng, 48)
        qc, sc = oracle.mxfp8_quant_row(np.ascontiguousarray(sample_cols(x, cols).T))
        assert np.array_equal(host(q["q_colT"][torch.as_tensor(cols, device="cuda")]), qc), name
        assert np.array_equal(scale_rows(q["s_colT"], cols), sc), name


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_dense_full_gemm_sampled(dense_full, which):
    rng = np.random.default_rng({"fwd": 1, "dgrad": 2, "wgrad": 3}[which])
    X, W, dY = dense_full["X"], dense_full["W"], dense_full["dY"]
    if which == "fwd":        # Y = X W : rows of X, columns of W
        out = dense_full["Y"]
        mi = boundary_indices(out.shape[0], 256, rng, 96)
        ni = boundary_indices(out.shape[1], 256, rng, 96)
        A, sA = oracle.mxfp8_quant_row(sample_rows(X, mi))
        B, sB = oracle.mxfp8_quant_row(np.ascontiguousarray(sample_cols(W, ni).T))
    elif which == "dgrad":    # dX = dY W^T : rows of dY, rows of W (along N)
        out = dense_full["dX"]
        mi = boundary_indices(out.shape[0], 256, rng, 96)
        ni = boundary_indices(out.shape[1], 256, rng, 96)
        A, sA = oracle.mxfp8_quant_row(sample_rows(dY, mi))
        B, sB = oracle.mxfp8_quant_row(sample_rows(W, ni))
    else:                     # dW = X^T dY : columns of X, columns of dY (along tokens)
        out = dense_full["dW"]
        mi = boundary_indices(out.shape[0], 256, rng, 96)
        ni = boundary_indices(out.shape[1], 256, rng, 96)
        A, sA = oracle.mxfp8_quant_row(np.ascontiguousarray(sample_cols(X, mi).T))
        B, sB = oracle.mxfp8_quant_row(np.ascontiguousarray(sample_cols(dY, ni).T))
    Cr, Ca = oracle.gemm(A, sA, B, sB)
    got = host(out[torch.as_tensor(mi, device="cuda")][:, torch.as_tensor(ni, device="cuda")])
    ratio = assert_gemm_close(got, Cr, Ca, f"dense {which}")
    print(f"dense {which}: {Cr.size} sampled outputs, max err/sum|ab| = {ratio:.3e}")
