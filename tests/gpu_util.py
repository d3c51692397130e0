"""Helpers shared by the GPU parity tests (imported only by tests marked gpu)."""
import numpy as np
import torch

import oracle
from moe_grouped_gemm_mxq_amd.workloads import bf16_bits

GEMM_TOL = 1e-5   # |err| <= GEMM_TOL * sum_k |a_k b_k| per element (fp32 accumulation)


def mxq():
    from moe_grouped_gemm_mxq_amd import mxq as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return m


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def unpack_scales(s: torch.Tensor, rows: int) -> np.ndarray:
    """GEMM-operand scale array of shape (ceil128(rows)/128, nblk, 32, 4)
    (element [r//128, b, r%32, (r//32)%4] = scale of row r, block b) ->
    row-major [rows][nblk] on the host."""
    q, nblk, b, i = s.shape
    assert b == 32 and i == 4 and q * 128 >= rows > q * 128 - 128, (tuple(s.shape), rows)
    return host(s.permute(0, 3, 2, 1).reshape(q * 128, nblk)[:rows])


def scale_rows(s: torch.Tensor, idx) -> np.ndarray:
    """Rows `idx` of a GEMM-operand scale array, row-major [len(idx)][nblk] on the host."""
    i = torch.as_tensor(np.asarray(idx), device=s.device)
    return host(s[i // 128, :, i % 32, (i // 32) % 4])


def out_host(got: dict, key: str, rows: int) -> np.ndarray:
    """A quantiser output on the host in the oracle's layout (scales unpacked)."""
    return unpack_scales(got[key], rows) if key.startswith("s_") else host(got[key])


def bits(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 bit patterns on the host."""
    return bf16_bits(x)


def scaled_randn(shape, seed, lo=-20, hi=20, zero_rows=0, axis=0):
    """N(0,1) bf16 times a random power of two per row (axis=0) or per column
    (axis=1), plus some all-zero rows.  Scaling whole reduction vectors keeps
    the within-block value distribution of the N(0,1) workloads."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    if axis == 0:
        x = x * torch.exp2(torch.randint(lo, hi, (shape[0], 1), generator=g).float())
    else:
        x = x * torch.exp2(torch.randint(lo, hi, (1, shape[1]), generator=g).float())
    if zero_rows:
        x[torch.randperm(shape[0], generator=g)[:zero_rows]] = 0.0
    return x.to(torch.bfloat16)


def mfma_group_bound(A, sA, B, sB, mi=None, ni=None):
    """Error model of the gfx950 FP8 scaled MFMA's internal summation on the
    plain (non-interleaved) path: it adds each group of 8 consecutive-K
    products with about 13 bits below the group's largest product
    (measured), so per output |err| <= 2^-10 * sum over groups of max
    |product| on top of fp32 rounding.  Used only by the test that documents
    this deviation on adversarial data; every parity test asserts the strict
    bound alone."""
    a = oracle.mxfp8_dequant(A, sA)
    b = oracle.mxfp8_dequant(B, sB)
    if mi is not None:
        a = a[mi]
    if ni is not None:
        b = b[ni]
    M, K = a.shape
    N = b.shape[0]
    ga = np.abs(a).reshape(M, K // 8, 8)
    gb = np.abs(b).reshape(N, K // 8, 8)
    out = np.zeros((M, N))
    for j in range(K // 8):
        out += np.max(ga[:, j, None, :] * gb[None, :, j, :], axis=2)
    return 2.0 ** -10 * out


def assert_gemm_close(got: np.ndarray, ref: np.ndarray, refabs: np.ndarray, what: str):
    """|got - ref| <= 1e-5 * sum_k |a_k b_k| for every output, no NaN/Inf.
    Returns max err / sum|ab| (the strict ratio)."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    err = np.abs(got - ref)
    bad = err > GEMM_TOL * refabs
    ratio = float(np.max(err / np.where(refabs > 0, refabs, 1.0))) if err.size else 0.0
    print(f"[strict] {what}: {err.size} outputs, max err/sum|ab| = {ratio:.3e} "
          f"({ratio / GEMM_TOL:.3f} of the bound)")
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outputs outside 1e-5*sum|ab|; "
                           f"max err/sum|ab| = {ratio:.3e}")
    return ratio


def deq(q, s) -> np.ndarray:
    """Oracle dequantisation of oracle codes and row-major scales (fp64)."""
    return oracle.mxfp8_dequant(np.ascontiguousarray(q), np.ascontiguousarray(s))


def boundary_indices(n: int, tile: int, rng, extra: int) -> np.ndarray:
    """Tile-boundary indices (first/last of every few tiles) plus random ones."""
    idx = {0, n - 1}
    for t0 in range(0, n, tile):
        idx.update({t0, min(t0 + tile - 1, n - 1)})
    idx = sorted(i for i in idx if 0 <= i < n)
    if len(idx) > extra:
        idx = list(rng.choice(idx, extra, replace=False))
    idx += list(rng.integers(0, n, extra))
    return np.unique(np.asarray(idx, np.int64))


def assert_bytes_equal(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    if np.array_equal(got, ref):
        return
    bad = np.argwhere(got != ref)
    if len(bad):
        ex = [(tuple(int(i) for i in b), int(got[tuple(b)]), int(ref[tuple(b)])) for b in bad[:8]]
        raise AssertionError(f"{what}: {len(bad)} of {got.size} bytes differ; first (index, got, want): {ex}")
