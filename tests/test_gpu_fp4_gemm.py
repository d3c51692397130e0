"""GPU parity of the MXFP4 GEMM operand quantiser and the E2M1 GEMMs against
the oracle (which quantises the same fp32 inputs itself)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_gemm_close, boundary_indices, host, mxq, unpack_scales

pytestmark = pytest.mark.gpu


def fp4_inputs(shape, seed, lo=-12, hi=12):
    """fp32 N(0,1) rows, each times a random power of two."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g) * torch.exp2(torch.randint(lo, hi, (shape[0], 1), generator=g).float())


def oracle_operand(x: torch.Tensor, sf: float = 6.0):
    _, codes, scales, _ = oracle.mxfp4_qdq_ex(x.numpy(), sf)
    return codes, scales


@pytest.mark.parametrize("shape,sf", [((1, 32), 6.0), ((5, 64), 6.0), ((33, 96), 5.0), ((70, 45), 6.0),
                                      ((300, 4096), 6.0), ((64, 160), 0.75)])
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


def test_gemm_fp4_full_size_sampled():
    """The dense linear's forward shape, M 8192 x N 18432 x K 7168, in MXFP4."""
    m = mxq()
    M, N, K = 8192, 18432, 7168
    g = torch.Generator(device="cuda").manual_seed(0)
    xa = torch.randn(M, K, generator=g, device="cuda")
    xb = torch.randn(N, K, generator=g, device="cuda") * 0.02
    qa, sa = m.quantize_fp4(xa)
    qb, sb = m.quantize_fp4(xb)
    C = m.gemm(qa, sa, qb, sb, fmt=m.MXQ_FMT_E2M1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    mi = boundary_indices(M, 256, rng, 24)
    ni = boundary_indices(N, 256, rng, 24)
    ra = host(xa[torch.as_tensor(mi, device="cuda")])
    rb = host(xb[torch.as_tensor(ni, device="cuda")])
    ca, csa = oracle_operand(torch.from_numpy(ra))
    cb, csb = oracle_operand(torch.from_numpy(rb))
    Cr, Ca = oracle.gemm_fp4(ca, csa, cb, csb)
    got = host(C[torch.as_tensor(mi, device="cuda")][:, torch.as_tensor(ni, device="cuda")])
    ratio = assert_gemm_close(got, Cr, Ca, "fp4 gemm 8192x18432x7168")
    print(f"fp4 gemm full size: {got.size} sampled outputs, max err/sum|ab| = {ratio:.3e}")


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
