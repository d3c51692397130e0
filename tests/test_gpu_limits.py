"""Largest sizes.  The quantisers past 2^31 elements (64-bit output
offsets; sampled rows and columns against the oracle), and the GEMMs at the
largest reduction length their tile addressing allows: code
rows of MXQ_GEMM_MAX_ROW_BYTES - 32 bytes, K = 2^23 - 32 for E4M3 and
2^24 - 32 for E2M1 (a 256-row tile of 2 GiB of codes).

The operands are built so that the exact result is known in closed form and
every partial sum is exact in fp32, whatever the summation order:
  * E4M3: A[i][k] = s_a(i, k) * m(i, k/32) with signs s_a = +-1 varying
    inside each block and block magnitudes m in {1, 2}; B[j][k] = s_b(j, k).
    Every code is exact (each block holds +-m), products are +-1 or +-2, and
    |sums| <= 2K < 2^24, so C must equal sum_k A B exactly.
  * E2M1: the same signs and magnitudes, but row i of A is nonzero only at
    k = i (mod 32); the block rule maps m to the scale 2^(round(log2(m/6))),
    so each nonzero dequantises to +-0.75 m and each B element to +-0.75:
    products are multiples of 9/16 whose running sums stay below 2^20.
The patterns have periods 11, 7, 32 and 96 along K (7392 in all), so the
closed form is a period's product times the number of periods plus the
remainder's, in float64.  A code or scale read from a wrong row, column or
block anywhere along the 2 GiB rows changes the result."""
import numpy as np
import pytest
import torch

from gpu_util import host, mxq


M = N = 256
PERIOD = 7392  # lcm(11, 7, 32, 96)


def sign_a(i, k):
    return np.where((k * 7 + i * 13) % 11 < 5, -1, 1)


def mag_a(i, k):
    return np.where(((k // 32) * 5 + i) % 3 == 0, 2, 1)


def sign_b(j, k):
    return np.where((k * 3 + j * 5) % 7 < 3, -1, 1)


def values(K, fp4, rows_a):
    """Dequantised operands over columns [0, K) on the host (float64)."""
    k = np.arange(K, dtype=np.int64)[None, :]
    i = np.arange(rows_a, dtype=np.int64)[:, None]
    j = np.arange(N, dtype=np.int64)[:, None]
    a = (sign_a(i, k) * mag_a(i, k)).astype(np.float64)
    b = sign_b(j, k).astype(np.float64)
    if fp4:
        a = np.where(k % 32 == i % 32, a * 0.75, 0.0)
        b = b * 0.75
    return a, b


def closed_form(K, fp4):
    q, r = divmod(K, PERIOD)
    a, b = values(PERIOD, fp4, M)
    c = q * (a @ b.T)
    if r:
        c += a[:, :r] @ b[:, :r].T
    return c


def build_on_gpu(K, fp4, dtype):
    """A [M][K] and B [N][K] on the GPU in `dtype`, a few rows at a time."""
    dev = torch.device("cuda")
    k = torch.arange(K, dtype=torch.int64, device=dev)[None, :]
    A = torch.empty((M, K), dtype=dtype, device=dev)
    B = torch.empty((N, K), dtype=dtype, device=dev)
    for r0 in range(0, M, 16):
        i = torch.arange(r0, r0 + 16, dtype=torch.int64, device=dev)[:, None]
        s = torch.where((k * 7 + i * 13) % 11 < 5, -1, 1)
        m = torch.where(((k // 32) * 5 + i) % 3 == 0, 2, 1)
        a = s * m
        if fp4:
            a = torch.where(k % 32 == i % 32, a, 0)
        A[r0:r0 + 16] = a.to(dtype)
        B[r0:r0 + 16] = torch.where((k * 3 + i * 5) % 7 < 3, -1, 1).to(dtype)
        del s, m, a
    return A, B


def test_closed_form_matches_the_definition_on_a_short_k():
    """The periodic closed form equals the plain product on a K that is not
    a multiple of the period (a host check of the test's own arithmetic)."""
    for fp4 in (False, True):
        K = 2 * PERIOD + 1000
        a, b = values(K, fp4, M)
        assert np.array_equal(closed_form(K, fp4), a @ b.T)


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_gemm_at_the_largest_k(fmt):
    m = mxq()
    fp4 = fmt == "e2m1"
    K = 2 * m.MAX_ROW_BYTES - 32 if fp4 else m.MAX_ROW_BYTES - 32
    print(f"[limits] {fmt} M={M} N={N} K={K}", flush=True)
    ref = closed_form(K, fp4)
    assert np.abs(ref).max() < (2 ** 20 if fp4 else 2 ** 24)   # every partial sum is exact in fp32
    A, B = build_on_gpu(K, fp4, torch.float32 if fp4 else torch.bfloat16)
    if fp4:
        qa, sa = m.quantize_fp4(A)
        del A
        qb, sb = m.quantize_fp4(B)
        del B
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        m.mxq_gemm(qa, sa, qb, sb, C, fmt=m.MXQ_FMT_E2M1)
    else:
        qa = m.quantize(A, m.MXQ_AXIS_ROW)
        del A
        qb = m.quantize(B, m.MXQ_AXIS_ROW)
        del B
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        m.mxq_gemm(qa["q_row"], qa["s_row"], qb["q_row"], qb["s_row"], C)
    got = host(C).astype(np.float64)
    assert np.array_equal(got, ref), f"max |diff| {np.abs(got - ref).max()}"


def _randn_bf16(R, C, seed):
    """N(0,1) bf16 [R][C] on the GPU, every 64th row and 48th column scaled by
    a power of two (so blocks of very different scales meet), a few rows at a time."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    col_scale = torch.where(torch.arange(C, device="cuda") % 48 == 5, 2.0 ** 20, 1.0)
    for r0 in range(0, R, 4096):
        r1 = min(R, r0 + 4096)
        row_scale = torch.where(torch.arange(r0, r1, device="cuda")[:, None] % 64 == 3, 2.0 ** -30, 1.0)
        x[r0:r1] = (torch.randn((r1 - r0, C), generator=g, device="cuda") * row_scale * col_scale).to(torch.bfloat16)
    return x


def _bits(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


@pytest.mark.gpu
def test_dual_quantise_beyond_2_31_elements():
    """Row and column copies of a 65536 x 36864 bf16 matrix (2.4e9 elements,
    output offsets past 2^31) in one dual-axis launch: sampled rows and
    columns, at the ends of the matrix and of its 128-row scale groups, equal
    the oracle's bytes."""
    import oracle
    from gpu_util import scale_rows
    m = mxq()
    R, C = 65536, 36864
    print(f"[limits] dual quantise {R}x{C}", flush=True)
    x = _randn_bf16(R, C, 11)
    got = m.quantize(x, m.MXQ_AXIS_ROW | m.MXQ_AXIS_COLT)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 3, 127, 128, 32767, 32768, 65411, 65535])
    cols = np.array([0, 5, 31, 32, 127, 128, 18431, 36805, 36863])
    q, s = oracle.mxfp8_quant_row(_bits(x[torch.as_tensor(rows, device="cuda")]))
    assert np.array_equal(host(got["q_row"][torch.as_tensor(rows, device="cuda")]), q)
    assert np.array_equal(scale_rows(got["s_row"], rows), s)
    qt, st = oracle.mxfp8_quant_colT(_bits(x[:, torch.as_tensor(cols, device="cuda")]))
    assert np.array_equal(host(got["q_colT"][torch.as_tensor(cols, device="cuda")]), qt)
    assert np.array_equal(scale_rows(got["s_colT"], cols), st)


@pytest.mark.gpu
def test_grouped_quantise_beyond_2_31_elements():
    """Token-axis copy (row copy too) of 131072 x 32768 bf16 in 32 groups of
    the MoE layer's sizes (4.3e9 elements; column-copy offsets past 2^32):
    sampled columns and rows equal the oracle's bytes."""
    import oracle
    from gpu_util import scale_rows
    from moe_grouped_gemm_mxq_amd import workloads
    m = mxq()
    T, C = 131072, 32768
    print(f"[limits] grouped quantise {T}x{C}", flush=True)
    sizes = workloads.moe_group_sizes()
    ge_np = np.cumsum(sizes).astype(np.int32)
    ge = torch.from_numpy(ge_np).cuda()
    x = _randn_bf16(T, C, 12)
    got = m.quantize_grouped(x, ge, m.MXQ_AXIS_ROW | m.MXQ_AXIS_COLT)
    torch.cuda.synchronize()
    cols = np.array([0, 5, 31, 127, 128, 16383, 32709, 32767])
    qt, st = oracle.mxfp8_quant_grouped_colT(_bits(x[:, torch.as_tensor(cols, device="cuda")]), ge_np, got["ldq"])
    P = oracle.grouped_cols(ge_np)   # positions past the groups' padded columns are not written
    assert np.array_equal(host(got["q_colT"][torch.as_tensor(cols, device="cuda")])[:, :P], qt[:, :P])
    assert np.array_equal(scale_rows(got["s_colT"], cols)[:, :P // 32], st[:, :P // 32])
    rows = np.array([0, 3, 65535, 131071])
    q, s = oracle.mxfp8_quant_row(_bits(x[torch.as_tensor(rows, device="cuda")]))
    assert np.array_equal(host(got["q_row"][torch.as_tensor(rows, device="cuda")]), q)
    assert np.array_equal(scale_rows(got["s_row"], rows), s)
