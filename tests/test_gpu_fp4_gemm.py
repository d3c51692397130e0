"""GPU parity of the MXFP4 GEMM operand quantiser and the E2M1 GEMMs against
the oracle (which quantises the same fp32 inputs itself)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_gemm_close, host, mxq, unpack_scales

pytestmark = pytest.mark.gpu


def fp4_inputs(shape, seed, lo=-12, hi=12):
    """fp32 N(0,1) rows, each times a random power of two."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g) * torch.exp2(torch.randint(lo, hi, (shape[0], 1), generator=g).float())


def oracle_operand(x: torch.Tensor, sf: float = 6.0):
    _, codes, scales, _ = oracle.mxfp4_qdq_ex(x.numpy(), sf)
    return codes, scales


@pytest.mark.parametrize("shape,sf", [((1, 32), 6.0), ((5, 64), 6.0), ((33, 96), 5.0), ((70, 45), 6.0),
                                      ((300, 4096), 6.0), ((64, 160), 0.75),
                                      # rows of a multiple of 1024 elements: 1024-element pieces,
                                      # two per workgroup (odd counts, partial 128-row groups,
                                      # full runs of eight groups and a tail)
                                      ((3, 1024), 6.0), ((129, 3072), 5.0), ((1029, 1024), 6.0),
                                      ((2053, 3072), 0.75)])
def test_quantize_fp4_matches_oracle(shape, sf):
    m = mxq()
    x = fp4_inputs(shape, sum(shape))
    codes, scales = m.quantize_fp4(x.cuda(), sf)
    torch.cuda.synchronize()
    rc, rs = oracle_operand(x, sf)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(unpack_scales(scales, shape[0]), rs)


def test_quantize_fp4_unaligned_input_takes_general_path():
    m = mxq()
    x = fp4_inputs((40, 128), 9)
    base = torch.empty(40 * 128 + 1, device="cuda")
    base[1:] = x.reshape(-1).cuda()
    codes, scales = m.quantize_fp4(base[1:].view(40, 128))
    torch.cuda.synchronize()
    rc, rs = oracle_operand(x)
    assert np.array_equal(host(codes), rc) and np.array_equal(unpack_scales(scales, 40), rs)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (300, 280, 96), (256, 256, 4096), (513, 70, 160), (40, 600, 4128)])
def test_gemm_fp4_matches_oracle(M, N, K):
    m = mxq()
    xa, xb = fp4_inputs((M, K), M + K), fp4_inputs((N, K), N + K + 1)
    qa, sa = m.quantize_fp4(xa.cuda())
    qb, sb = m.quantize_fp4(xb.cuda())
    C = m.gemm(qa, sa, qb, sb, fmt=m.MXQ_FMT_E2M1)
    torch.cuda.synchronize()
    ca, csa = oracle_operand(xa)
    cb, csb = oracle_operand(xb)
    Cr, Ca = oracle.gemm_fp4(ca, csa, cb, csb)
    assert_gemm_close(host(C), Cr, Ca, f"fp4 gemm {M}x{N}x{K}")


def test_gemm_fp4_full_size_every_output():
    """The dense linear's forward shape, M 8192 x N 18432 x K 7168, in MXFP4:
    every code and scale byte of both operands and every one of the 151M
    outputs against the oracle's fp64 product of its own dequantised codes."""
    m = mxq()
    M, N, K = 8192, 18432, 7168
    g = torch.Generator(device="cuda").manual_seed(0)
    xa = torch.randn(M, K, generator=g, device="cuda")
    xb = torch.randn(N, K, generator=g, device="cuda") * 0.02
    qa, sa = m.quantize_fp4(xa)
    qb, sb = m.quantize_fp4(xb)
    C = m.gemm(qa, sa, qb, sb, fmt=m.MXQ_FMT_E2M1)
    torch.cuda.synchronize()
    ca, csa = oracle_operand(torch.from_numpy(host(xa)))
    del xa
    assert np.array_equal(host(qa), ca) and np.array_equal(unpack_scales(sa, M), csa)
    cb, csb = oracle_operand(torch.from_numpy(host(xb)))
    del xb
    assert np.array_equal(host(qb), cb) and np.array_equal(unpack_scales(sb, N), csb)
    Cr, Ca = oracle.gemm_dequantised(oracle.mxfp4_dequant(ca, csa, K), oracle.mxfp4_dequant(cb, csb, K))
    ratio = assert_gemm_close(host(C), Cr, Ca, "fp4 gemm 8192x18432x7168 (every output)")
    print(f"fp4 gemm full size: every output, max err/sum|ab| = {ratio:.3e}")


def test_grouped_gemm_fp4_ragged_m_moe_every_output():
    """The MoE forward shape in MXFP4: fp32 token rows X [131072x7168] N(0,1)
    grouped by the frozen Zipf(1.1) routing, expert weights W[g] [4096x7168]
    N(0, 0.02^2); every output of Y [131072x4096], expert by expert."""
    from moe_grouped_gemm_mxq_amd import workloads
    m = mxq()
    sizes = workloads.moe_group_sizes()
    ge_np = np.cumsum(sizes).astype(np.int32)
    ge = torch.from_numpy(ge_np).cuda()
    G, N, K, T = len(sizes), 4096, 7168, int(ge_np[-1])
    g = torch.Generator(device="cuda").manual_seed(4)
    X = torch.randn(T, K, generator=g, device="cuda")
    W = torch.randn(G, N, K, generator=g, device="cuda") * 0.02
    qx, sx = m.quantize_fp4(X)
    qw = torch.empty((G, N, K // 2), dtype=torch.uint8, device="cuda")
    sw = torch.empty((G,) + m.scale_shape(N, K // 32), dtype=torch.uint8, device="cuda")
    for e in range(G):
        m.mxq_quantize_fp4(W[e], qw[e], sw[e])
    Y = m.grouped_gemm(m.MXQ_GG_RAGGED_M, qx, sx, qw, sw, ge, fmt=m.MXQ_FMT_E2M1)
    torch.cuda.synchronize()
    xc, xs = oracle_operand(torch.from_numpy(host(X)))
    del X
    assert np.array_equal(host(qx), xc) and np.array_equal(unpack_scales(sx, T), xs)
    out = host(Y)
    worst, start = 0.0, 0
    for e, end in enumerate(ge_np.tolist()):
        wc, ws = oracle_operand(torch.from_numpy(host(W[e])))
        assert np.array_equal(host(qw[e]), wc) and np.array_equal(unpack_scales(sw[e], N), ws)
        if end > start:
            Cr, Ca = oracle.gemm_dequantised(oracle.mxfp4_dequant(xc[start:end], xs[start:end], K),
                                             oracle.mxfp4_dequant(wc, ws, K))
            worst = max(worst, assert_gemm_close(out[start:end], Cr, Ca,
                                                 f"fp4 moe fwd expert {e} ({end - start} rows)"))
        start = end
    print(f"fp4 moe fwd: every output, max err/sum|ab| = {worst:.3e}")


@pytest.mark.parametrize("sizes", [[5, 0, 300, 33], [256, 1, 0, 0, 513]])
@pytest.mark.parametrize("K", [192, 608])
def test_grouped_gemm_fp4_ragged_m(sizes, K):
    m = mxq()
    T, N, G = sum(sizes), 96, len(sizes)
    x = fp4_inputs((T, K), T + 7)
    w = fp4_inputs((G * N, K), T + 8)
    ge_np = np.cumsum(sizes).astype(np.int32)
    ge = torch.from_numpy(ge_np).cuda()
    qa, sa = m.quantize_fp4(x.cuda())
    qw = torch.empty((G, N, K // 2), dtype=torch.uint8, device="cuda")
    sw = torch.empty((G,) + m.scale_shape(N, K // 32), dtype=torch.uint8, device="cuda")
    wd = w.cuda()
    for g in range(G):
        m.mxq_quantize_fp4(wd[g * N:(g + 1) * N], qw[g], sw[g])
    C = torch.full((T + 3, N), 3.0, device="cuda")    # 3 rows past the groups stay untouched
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_M, qa, sa, qw, sw, C[:T], ge, fmt=m.MXQ_FMT_E2M1)
    torch.cuda.synchronize()
    ca, csa = oracle_operand(x)
    got = host(C)
    start = 0
    for g, s in enumerate(sizes):
        if s:
            cw, csw = oracle_operand(w[g * N:(g + 1) * N])
            Cr, Ca = oracle.gemm_fp4(ca[start:start + s], csa[start:start + s], cw, csw)
            assert_gemm_close(got[start:start + s], Cr, Ca, f"fp4 ragged M group {g}")
        start += s
    assert np.all(got[T:] == 3.0)


# ------------------------------------------------------------------ grouped token axis (expert weight gradient)
def grouped_fp4_case(sizes, C, seed, sf=6.0):
    m = mxq()
    T = sum(sizes)
    x = fp4_inputs((T, C), seed)
    ge_np = np.cumsum(sizes).astype(np.int32)
    ge = torch.from_numpy(ge_np).cuda()
    q = m.quantize_fp4_grouped(x.cuda(), ge, scale_factor=sf)
    torch.cuda.synchronize()
    rc, rs = oracle.mxfp4_quant_grouped_colT(x.numpy(), ge_np, q["ldq"], sf)
    return q, rc, rs, ge_np


@pytest.mark.parametrize("sizes,C,sf", [([5, 0, 33, 1, 257, 64], 70, 6.0), ([0, 0, 300], 32, 6.0),
                                        ([1], 1, 6.0), ([31, 32, 33, 0, 513], 200, 5.0),
                                        ([0, 31, 0, 32, 0, 33, 512, 0], 96, 7.25)])
def test_quantize_fp4_grouped_bitexact(sizes, C, sf):
    q, rc, rs, ge_np = grouped_fp4_case(sizes, C, sum(sizes) + C, sf)
    P = oracle.grouped_cols(ge_np)
    assert np.array_equal(host(q["codes"])[:, :P // 2], rc[:, :P // 2])
    assert np.array_equal(unpack_scales(q["scales"], C)[:, :P // 32], rs[:, :P // 32])


def test_quantize_fp4_grouped_unaligned_input():
    """A row pitch that is not a multiple of 4 floats takes the scalar loads."""
    m = mxq()
    sizes, C = [40, 0, 77], 45
    T = sum(sizes)
    x = fp4_inputs((T, C), 3)
    base = torch.zeros((T, C + 1), device="cuda")
    base[:, :C] = x.cuda()
    ge_np = np.cumsum(sizes).astype(np.int32)
    q = m.quantize_fp4_grouped(base[:, :C], torch.from_numpy(ge_np).cuda())
    torch.cuda.synchronize()
    rc, rs = oracle.mxfp4_quant_grouped_colT(x.numpy(), ge_np, q["ldq"])
    P = oracle.grouped_cols(ge_np)
    assert np.array_equal(host(q["codes"])[:, :P // 2], rc[:, :P // 2])
    assert np.array_equal(unpack_scales(q["scales"], C)[:, :P // 32], rs[:, :P // 32])


def check_fp4_wgrad(dW, xc, xs, yc, ys, ge_np, what):
    """Every output of every expert against the oracle's fp64 product of the
    dequantised codes; empty experts exact zeros."""
    start, P = 0, 0
    for g, e in enumerate(np.asarray(ge_np).tolist()):
        w = oracle.ceil32(e - start)
        if w == 0:
            assert not dW[g].any(), f"{what}: empty expert {g} has nonzero dW"
        else:
            a = oracle.mxfp4_dequant(np.ascontiguousarray(xc[:, P // 2:(P + w) // 2]),
                                     np.ascontiguousarray(xs[:, P // 32:(P + w) // 32]), w)
            b = oracle.mxfp4_dequant(np.ascontiguousarray(yc[:, P // 2:(P + w) // 2]),
                                     np.ascontiguousarray(ys[:, P // 32:(P + w) // 32]), w)
            Cr, Ca = oracle.gemm_dequantised(a, b)
            assert_gemm_close(dW[g], Cr, Ca, f"{what} expert {g} ({e - start} tokens)")
        P += w
        start = e


@pytest.mark.parametrize("sizes", [[5, 0, 33, 1, 257, 64], [0, 0, 300], [513, 4, 1024, 0, 1500], [1]])
def test_grouped_gemm_fp4_ragged_k(sizes):
    m = mxq()
    qx, xc, xs, ge_np = grouped_fp4_case(sizes, 70, sum(sizes) + 1)
    qy, yc, ys, _ = grouped_fp4_case(sizes, 90, sum(sizes) + 2)
    ge = torch.from_numpy(ge_np).cuda()
    dW = m.grouped_gemm(m.MXQ_GG_RAGGED_K, qx["codes"], qx["scales"], qy["codes"], qy["scales"], ge,
                        fmt=m.MXQ_FMT_E2M1)
    torch.cuda.synchronize()
    check_fp4_wgrad(host(dW), xc, xs, yc, ys, ge_np, f"fp4 ragged K {sizes}")


def test_grouped_gemm_fp4_ragged_k_moe_every_output():
    """The MoE weight-gradient shape in MXFP4: fp32 token rows X [131072x7168]
    and dY [131072x4096], N(0,1), grouped by the frozen Zipf(1.1) routing;
    every output of all 32 experts' dW [7168x4096]."""
    from moe_grouped_gemm_mxq_amd import workloads
    m = mxq()
    sizes = workloads.moe_group_sizes()
    ge_np = np.cumsum(sizes).astype(np.int32)
    ge = torch.from_numpy(ge_np).cuda()
    g = torch.Generator(device="cuda").manual_seed(3)
    T = int(ge_np[-1])
    X = torch.randn(T, 7168, generator=g, device="cuda")
    dY = torch.randn(T, 4096, generator=g, device="cuda")
    qx = m.quantize_fp4_grouped(X, ge)
    qy = m.quantize_fp4_grouped(dY, ge, ldq=qx["ldq"])
    dW = m.grouped_gemm(m.MXQ_GG_RAGGED_K, qx["codes"], qx["scales"], qy["codes"], qy["scales"], ge,
                        fmt=m.MXQ_FMT_E2M1)
    torch.cuda.synchronize()
    P = oracle.grouped_cols(ge_np)
    xc, xs = oracle.mxfp4_quant_grouped_colT(host(X), ge_np, qx["ldq"])
    assert np.array_equal(host(qx["codes"])[:, :P // 2], xc[:, :P // 2])
    assert np.array_equal(unpack_scales(qx["scales"], 7168)[:, :P // 32], xs[:, :P // 32])
    del X
    yc, ys = oracle.mxfp4_quant_grouped_colT(host(dY), ge_np, qx["ldq"])
    assert np.array_equal(host(qy["codes"])[:, :P // 2], yc[:, :P // 2])
    del dY
    check_fp4_wgrad(host(dW), xc, xs, yc, ys, ge_np, "fp4 moe wgrad")
