"""Seeded random-shape sweep of the GPU path against the oracle.  Shapes, K
tails, group counts and group sizes (with empty and tiny groups) are drawn at
random from fixed seeds, so tile tails, partial 128-row scale groups and
group boundaries meet in combinations the hand-picked cases do not.  Same
bars as the other parity tests: codes and scales bit-exact, GEMM outputs
within 1e-5 * sum|ab| (E2M1 outputs exact).  K is drawn on both sides of
the 1024-element interleaving threshold."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bytes_equal, assert_gemm_close, bits, host, mxq, out_host, scaled_randn, unpack_scales

pytestmark = pytest.mark.gpu
SEEDS = list(range(8))


def draw_sizes(rng, G, hi):
    sizes = rng.integers(0, hi, G)
    sizes[rng.random(G) < 0.25] = 0           # some empty groups
    sizes[rng.random(G) < 0.15] = 1           # and some single rows
    return sizes.astype(np.int64)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_quantize(seed):
    rng = np.random.default_rng(100 + seed)
    R, C = int(rng.integers(1, 700)), int(rng.integers(1, 700))
    axis = int(rng.integers(1, 4))
    x = scaled_randn((R, C), 100 + seed, zero_rows=int(rng.integers(0, 3)))
    got = mxq().quantize(x.cuda(), axis)
    torch.cuda.synchronize()
    xb = bits(x)
    ref = {}
    if axis & 1:
        ref["q_row"], ref["s_row"] = oracle.mxfp8_quant_row(xb)
    if axis & 2:
        ref["q_colT"], ref["s_colT"] = oracle.mxfp8_quant_colT(xb)
    for k, v in ref.items():
        assert_bytes_equal(out_host(got, k, v.shape[0]), v, f"{k} {R}x{C} axis {axis}")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_grouped_quantize(seed):
    rng = np.random.default_rng(200 + seed)
    G, C = int(rng.integers(1, 12)), int(rng.integers(1, 300))
    sizes = draw_sizes(rng, G, 200)
    T = int(sizes.sum())
    if T == 0:
        sizes[0], T = 7, 7
    x = scaled_randn((T, C), 200 + seed)
    ge = np.cumsum(sizes).astype(np.int32)
    got = mxq().quantize_grouped(x.cuda(), torch.from_numpy(ge).cuda(), 3)
    torch.cuda.synchronize()
    P = oracle.grouped_cols(ge)
    q, s = oracle.mxfp8_quant_grouped_colT(bits(x), ge, got["ldq"])
    assert_bytes_equal(host(got["q_colT"])[:, :P], q[:, :P], f"grouped colT codes {sizes.tolist()} x {C}")
    assert_bytes_equal(out_host(got, "s_colT", C)[:, :P // 32], s[:, :P // 32], "grouped colT scales")
    qr, sr = oracle.mxfp8_quant_row(bits(x))
    assert_bytes_equal(host(got["q_row"]), qr, "grouped row codes")
    assert_bytes_equal(out_host(got, "s_row", T), sr, "grouped row scales")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_dense_gemm(seed):
    rng = np.random.default_rng(300 + seed)
    M, N, K = int(rng.integers(1, 600)), int(rng.integers(1, 600)), int(rng.integers(1, 2000))
    m = mxq()
    X = scaled_randn((M, K), 300 + seed, lo=-8, hi=8)
    W = scaled_randn((N, K), 350 + seed, lo=-8, hi=8)
    qa, qb = m.quantize(X.cuda(), 1), m.quantize(W.cuda(), 1)
    C = m.gemm(qa["q_row"], qa["s_row"], qb["q_row"], qb["s_row"])
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_row(bits(X))
    B, sB = oracle.mxfp8_quant_row(bits(W))
    Cr, Ca = oracle.gemm(A, sA, B, sB)
    assert_gemm_close(host(C), Cr, Ca, f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_ragged_m(seed):
    rng = np.random.default_rng(400 + seed)
    G, N, K = int(rng.integers(1, 10)), int(rng.integers(1, 300)), int(rng.integers(1, 64)) * 32
    sizes = draw_sizes(rng, G, 400)
    T = int(sizes.sum())
    m = mxq()
    X = scaled_randn((T + 3, K), 400 + seed, lo=-6, hi=6)     # 3 trailing rows in no group
    W = scaled_randn((G * K, N), 450 + seed, lo=-6, hi=6, axis=1).reshape(G, K, N)
    ge = np.cumsum(sizes).astype(np.int32)
    qx = m.quantize(X.cuda(), 1)
    qw = m.quantize_batched(W.cuda(), 2)                      # B[g] = column copy of W[g]
    C = torch.full((T + 3, N), 3.0, device="cuda")
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_M, qx["q_row"], qx["s_row"], qw["q_colT"], qw["s_colT"], C,
                       torch.from_numpy(ge).cuda())
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_row(bits(X))
    refB = [oracle.mxfp8_quant_colT(bits(W[g])) for g in range(G)]
    Bq, Bs = np.stack([b[0] for b in refB]), np.stack([b[1] for b in refB])
    got = host(C)
    if T:
        Cr, Ca = oracle.grouped_gemm_ragged_m(A, sA, Bq, Bs, ge)
        assert_gemm_close(got[:T], Cr[:T], Ca[:T], f"ragged M {sizes.tolist()} N {N} K {K}")
    assert np.all(got[T:] == 3.0), "rows in no group were written"


@pytest.mark.parametrize("seed", SEEDS)
def test_random_ragged_k(seed):
    rng = np.random.default_rng(500 + seed)
    G, Mh, N = int(rng.integers(1, 10)), int(rng.integers(1, 300)), int(rng.integers(1, 300))
    sizes = draw_sizes(rng, G, 2000)
    if sizes.sum() == 0:
        sizes[-1] = 5
    T = int(sizes.sum())
    m = mxq()
    X = scaled_randn((T, Mh), 500 + seed, lo=-6, hi=6, axis=1)
    dY = scaled_randn((T, N), 550 + seed, lo=-6, hi=6, axis=1)
    ge_np = np.cumsum(sizes).astype(np.int32)
    ge = torch.from_numpy(ge_np).cuda()
    qx = m.quantize_grouped(X.cuda(), ge, 2)
    qy = m.quantize_grouped(dY.cuda(), ge, 2, ldq=qx["ldq"])
    C = m.grouped_gemm(m.MXQ_GG_RAGGED_K, qx["q_colT"], qx["s_colT"], qy["q_colT"], qy["s_colT"], ge)
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_grouped_colT(bits(X), ge_np, qx["ldq"])
    B, sB = oracle.mxfp8_quant_grouped_colT(bits(dY), ge_np, qx["ldq"])
    Cr, Ca = oracle.grouped_gemm_ragged_k(A, sA, B, sB, ge_np)
    got = host(C)
    assert_gemm_close(got, Cr, Ca, f"ragged K {sizes.tolist()} {Mh}x{N}")
    for g, s in enumerate(sizes.tolist()):
        if s == 0:
            assert np.all(got[g] == 0.0), f"empty group {g} not exactly zero"


@pytest.mark.parametrize("seed", SEEDS)
def test_random_fp4_qdq_and_gemm(seed):
    rng = np.random.default_rng(600 + seed)
    rows, L = int(rng.integers(1, 300)), int(rng.integers(1, 500))
    sf = float(np.float32(rng.choice([6.0, 5.0, 4.5, 7.25, 3.0, 12.0])))
    g = torch.Generator().manual_seed(600 + seed)
    x = torch.randn(rows, L, generator=g) * torch.exp2(torch.randint(-20, 20, (rows, 1), generator=g).float())
    m = mxq()
    y, mask = m.qdq_fp4_ste(x.cuda(), sf)
    torch.cuda.synchronize()
    ry, _, _, rm = oracle.mxfp4_qdq_ex(x.numpy(), sf)
    assert np.array_equal(host(y).view(np.uint32), ry.view(np.uint32)), f"QDQ {rows}x{L} sf {sf}"
    assert np.array_equal(host(mask), rm), f"saturation mask {rows}x{L} sf {sf}"
    # the FP4 GEMM of two such operands (K = L padded to 32)
    N = int(rng.integers(1, 200))
    w = torch.randn(N, L, generator=g)
    qa, sa = m.quantize_fp4(x.cuda())
    qb, sb = m.quantize_fp4(w.cuda())
    C = m.gemm(qa, sa, qb, sb, fmt=m.MXQ_FMT_E2M1)
    torch.cuda.synchronize()
    _, ca, s_a, _ = oracle.mxfp4_qdq_ex(x.numpy(), 6.0)
    _, cb, s_b, _ = oracle.mxfp4_qdq_ex(w.numpy(), 6.0)
    Cr, Ca = oracle.gemm_fp4(ca, s_a, cb, s_b)
    assert_gemm_close(host(C), Cr, Ca, f"FP4 GEMM {rows}x{N}x{L}")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_fp4_operand_rows_of_whole_kilo_elements(seed):
    """MXFP4 GEMM operands of rows whose length is a multiple of 1024 (the
    row-piece kernel): random row counts (partial 128-row groups, odd piece
    counts) and scale factors, every code and scale byte against the oracle."""
    rng = np.random.default_rng(700 + seed)
    rows, L = int(rng.integers(1, 700)), 1024 * int(rng.integers(1, 6))
    sf = float(np.float32(rng.choice([6.0, 5.0, 7.25, 3.0])))
    g = torch.Generator().manual_seed(700 + seed)
    x = torch.randn(rows, L, generator=g) * torch.exp2(torch.randint(-20, 20, (rows, 1), generator=g).float())
    codes, scales = mxq().quantize_fp4(x.cuda(), sf)
    torch.cuda.synchronize()
    _, rc, rs, _ = oracle.mxfp4_qdq_ex(x.numpy(), sf)
    assert np.array_equal(host(codes), rc), f"codes {rows}x{L} sf {sf}"
    assert np.array_equal(unpack_scales(scales, rows), rs), f"scales {rows}x{L} sf {sf}"
