"""CPU oracle for MX microscaling quantisation and block-scaled GEMMs.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  The
arithmetic lives in ``mxq_oracle.c`` (plain C, fp64), compiled with gcc into
``liboracle.so`` next to this file; this module only marshals numpy arrays.

bf16 tensors are passed as ``uint16`` bit patterns (numpy has no bf16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BLOCK = 32


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _declare(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    sig = {
        "oracle_num_threads": ([], ctypes.c_int),
        "oracle_set_num_threads": ([ctypes.c_int], None),
        "oracle_e4m3_decode": ([ctypes.c_uint8], ctypes.c_double),
        "oracle_e4m3_encode": ([ctypes.c_double], ctypes.c_uint8),
        "oracle_e4m3_encode_n": ([P, I64, P], None),
        "oracle_e8m0_decode": ([ctypes.c_uint8], ctypes.c_double),
        "oracle_mxfp8_quant_row": ([P, I64, I64, I64, P, P], ctypes.c_int),
        "oracle_mxfp8_quant_colT": ([P, I64, I64, I64, P, P], ctypes.c_int),
        "oracle_mxfp8_quant_grouped_colT": ([P, I64, I64, I64, P, I32, I64, P, P], ctypes.c_int),
        "oracle_mxfp8_dequant": ([P, P, I64, I64, P], None),
        "oracle_mxfp4_qdq": ([P, P, I64, I64, P, P], ctypes.c_int),
        "oracle_mxfp4_qdq_ex": ([P, P, I64, I64, ctypes.c_float, P, P, P], ctypes.c_int),
        "oracle_mxfp4_ste_backward": ([P, P, P, I64, I64], None),
        "oracle_gemm": ([P, P, P, P, I64, I64, I64, P, P], ctypes.c_int),
        "oracle_mxfp4_dequant": ([P, P, I64, I64, P], None),
        "oracle_gemm_fp4": ([P, P, P, P, I64, I64, I64, P, P], ctypes.c_int),
        "oracle_gemm_fp4_sampled": ([P, P, P, P, I64, I64, I64, P, P, I64, P, P], ctypes.c_int),
        "oracle_gemm_sampled": ([P, P, P, P, I64, I64, I64, P, P, I64, P, P], ctypes.c_int),
        "oracle_grouped_gemm_ragged_m": ([P, P, P, P, I64, I64, I64, P, I32, P, P], ctypes.c_int),
        "oracle_grouped_gemm_ragged_m_sampled":
            ([P, P, P, P, I64, I64, I64, P, I32, P, P, I64, P, P], ctypes.c_int),
        "oracle_grouped_gemm_ragged_k": ([P, P, P, P, I64, I64, I64, P, I32, P, P], ctypes.c_int),
        "oracle_grouped_gemm_ragged_k_sampled":
            ([P, P, P, P, I64, I64, I64, P, I32, P, P, P, I64, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def lib(path: str | None = None):
    """Load the oracle library, compiling it first if it is not built."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


class using:
    """Context manager that routes this module's calls to another build of the
    oracle (the mutation tests use it to run the pins against planted bugs)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _declare(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (status {rc})")


def ceil32(v: int) -> int:
    return (v + BLOCK - 1) // BLOCK * BLOCK


def grouped_cols(group_end) -> int:
    """Columns used by a grouped token-axis copy: sum of ceil32(group sizes)."""
    prev, tot = 0, 0
    for e in np.asarray(group_end, dtype=np.int64).tolist():
        tot += ceil32(e - prev)
        prev = e
    return tot


# ---------------------------------------------------------------- elements
def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(float(v))


def e4m3_encode_array(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.zeros(v.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_p(v), v.size, _p(out))
    return out


def e8m0_decode(byte: int) -> float:
    return lib().oracle_e8m0_decode(int(byte))


# ---------------------------------------------------------------- MXFP8
def mxfp8_quant_row(x_bits: np.ndarray):
    """bf16 bits [R][C] -> (codes uint8 [R][Cp], scales uint8 [R][Cp/32])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    Cp = ceil32(C)
    q = np.zeros((R, Cp), np.uint8)
    s = np.zeros((R, Cp // BLOCK), np.uint8)
    _check(lib().oracle_mxfp8_quant_row(_p(x), R, C, C, _p(q), _p(s)), "quant_row")
    return q, s


def mxfp8_quant_colT(x_bits: np.ndarray):
    """bf16 bits [R][C] -> (codes [C][Rp], scales [C][Rp/32]) of the transpose."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    Rp = ceil32(R)
    q = np.zeros((C, Rp), np.uint8)
    s = np.zeros((C, Rp // BLOCK), np.uint8)
    _check(lib().oracle_mxfp8_quant_colT(_p(x), R, C, C, _p(q), _p(s)), "quant_colT")
    return q, s


def mxfp8_quant_grouped_colT(x_bits: np.ndarray, group_end, ldq: int | None = None):
    """bf16 bits [T][C] + cumulative group ends -> (codes [C][ldq], scales [C][ldq/32]).

    Columns at and beyond sum_g ceil32(m_g) are returned as zeros.
    """
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, C = x.shape
    ge = np.ascontiguousarray(group_end, dtype=np.int32)
    if ldq is None:
        ldq = max(grouped_cols(ge), BLOCK)
    q = np.zeros((C, ldq), np.uint8)
    s = np.zeros((C, ldq // BLOCK), np.uint8)
    _check(lib().oracle_mxfp8_quant_grouped_colT(_p(x), T, C, C, _p(ge), len(ge), ldq,
                                                 _p(q), _p(s)), "quant_grouped_colT")
    return q, s


def mxfp8_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    R, K = q.shape
    assert s.shape == (R, K // BLOCK)
    out = np.zeros((R, K), np.float64)
    lib().oracle_mxfp8_dequant(_p(q), _p(s), R, K, _p(out))
    return out


# ---------------------------------------------------------------- MXFP4
def mxfp4_qdq(x: np.ndarray, want_codes: bool = False):
    """fp32 array of any shape -> fp32 QDQ of the same shape (blocks of 32 on
    the last dim, each row padded on its own).  With ``want_codes`` also
    returns (codes [rows][Lp/2], scales [rows][Lp/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    shape = x.shape
    L = shape[-1] if x.ndim else 1
    rows = int(np.prod(shape[:-1])) if x.ndim > 1 else 1
    y = np.zeros(shape, np.float32)
    Lp = ceil32(L)
    codes = np.zeros((rows, Lp // 2), np.uint8) if want_codes else None
    scales = np.zeros((rows, Lp // BLOCK), np.uint8) if want_codes else None
    _check(lib().oracle_mxfp4_qdq(_p(x), _p(y), rows, L, _p(codes), _p(scales)), "mxfp4_qdq")
    return (y, codes, scales) if want_codes else y


def mxfp4_qdq_ex(x: np.ndarray, scale_factor: float = 6.0):
    """QDQ with a runtime scale factor (an fp32 value; the page's
    inv_scale_factor_scale is 6 / scale_factor).  Returns (y, codes [rows][Lp/2],
    scales [rows][Lp/32], saturation mask [rows][Lp/8], bit j of byte k =
    element 8k+j has |x| > 6*scale)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    shape = x.shape
    L = shape[-1] if x.ndim else 1
    rows = int(np.prod(shape[:-1])) if x.ndim > 1 else 1
    y = np.zeros(shape, np.float32)
    Lp = ceil32(L)
    codes = np.zeros((rows, Lp // 2), np.uint8)
    scales = np.zeros((rows, Lp // BLOCK), np.uint8)
    mask = np.zeros((rows, Lp // 8), np.uint8)
    _check(lib().oracle_mxfp4_qdq_ex(_p(x), _p(y), rows, L, float(np.float32(scale_factor)), _p(codes),
                                     _p(scales), _p(mask)), "mxfp4_qdq_ex")
    return y, codes, scales, mask


def mxfp4_ste_backward(grad_y: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Clipped-STE backward: grad_y where the element did not saturate, else 0."""
    grad_y = np.ascontiguousarray(grad_y, dtype=np.float32)
    L = grad_y.shape[-1]
    rows = grad_y.size // L
    gx = np.zeros_like(grad_y)
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    assert mask.shape == (rows, ceil32(L) // 8)
    lib().oracle_mxfp4_ste_backward(_p(grad_y), _p(mask), _p(gx), rows, L)
    return gx


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray, L: int) -> np.ndarray:
    """MXFP4 codes [rows][ceil32(L)/2] + row-major scales [rows][ceil32(L)/32] -> fp64 [rows][L]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    assert codes.shape == (rows, ceil32(L) // 2) and scales.shape == (rows, ceil32(L) // BLOCK)
    out = np.zeros((rows, L), np.float64)
    lib().oracle_mxfp4_dequant(_p(codes), _p(scales), rows, L, _p(out))
    return out


def gemm_fp4(A, sA, B, sB):
    """MXFP4 operands (codes [M][K/2], row-major scales [M][K/32]):
    C[m][n] = sum_k deq(A)[m][k]*deq(B)[n][k]; returns (C, sum|products|) in fp64."""
    A, sA, B, sB = (np.ascontiguousarray(t, dtype=np.uint8) for t in (A, sA, B, sB))
    M, K = A.shape[0], A.shape[1] * 2
    N = B.shape[0]
    assert sA.shape == (M, K // BLOCK) and B.shape == (N, K // 2) and sB.shape == (N, K // BLOCK)
    C = np.zeros((M, N), np.float64)
    Cabs = np.zeros((M, N), np.float64)
    _check(lib().oracle_gemm_fp4(_p(A), _p(sA), _p(B), _p(sB), M, N, K, _p(C), _p(Cabs)), "gemm_fp4")
    return C, Cabs


def gemm_fp4_sampled(A, sA, B, sB, mi, ni):
    A, sA, B, sB = (np.ascontiguousarray(t, dtype=np.uint8) for t in (A, sA, B, sB))
    M, K = A.shape[0], A.shape[1] * 2
    N = B.shape[0]
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    C = np.zeros(len(mi), np.float64)
    Cabs = np.zeros(len(mi), np.float64)
    _check(lib().oracle_gemm_fp4_sampled(_p(A), _p(sA), _p(B), _p(sB), M, N, K, _p(mi), _p(ni), len(mi),
                                         _p(C), _p(Cabs)), "gemm_fp4_sampled")
    return C, Cabs


def mxfp4_quant_grouped_colT(x: np.ndarray, group_end, ldq: int, scale_factor: float = 6.0):
    """MXFP4 blocks down the token axis of x fp32 [T][C] within each group
    (the weight-gradient operands of the MXFP4 expert GEMMs): group g's rows,
    transposed to [C][m_g], go through the MXFP4 quantiser above (row padding =
    the group's zero tail), and land at padded positions [P_g, P_g +
    ceil32(m_g)).  Returns codes [C][ldq/2] and row-major scales [C][ldq/32];
    positions at and past P_G are zero."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, C = x.shape
    ge = np.asarray(group_end, dtype=np.int64)
    assert ldq % BLOCK == 0 and grouped_cols(ge) <= ldq
    codes = np.zeros((C, ldq // 2), np.uint8)
    scales = np.zeros((C, ldq // BLOCK), np.uint8)
    start, P = 0, 0
    for e in ge.tolist():
        assert start <= e <= T, "group ends must be non-decreasing and <= T"
        m = e - start
        if m:
            _, cg, sg, _ = mxfp4_qdq_ex(np.ascontiguousarray(x[start:e].T), scale_factor)
            codes[:, P // 2:(P + ceil32(m)) // 2] = cg
            scales[:, P // BLOCK:(P + ceil32(m)) // BLOCK] = sg
        P += ceil32(m)
        start = e
    return codes, scales


# ---------------------------------------------------------------- GEMMs
def gemm_dequantised(a: np.ndarray, b: np.ndarray):
    """C = a b^T and sum_k |a_k b_k| = |a| |b|^T for operands already
    dequantised to fp64 (mxfp8_dequant / mxfp4_dequant rows of K values).

    The same definition as ``gemm`` -- fp64 sums of the exact products -- with
    numpy's fp64 matrix product as the summation step (only the order of the
    fp64 additions differs), for full-size checks where the plain loops take
    minutes."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    assert a.ndim == 2 and b.ndim == 2 and a.shape[1] == b.shape[1]
    C = a @ b.T
    Cabs = np.abs(a) @ np.abs(b).T
    return C, Cabs


def gemm(A, sA, B, sB):
    """C[m][n] = sum_k deq(A)[m][k]*deq(B)[n][k]; returns (C, sum|products|) in fp64."""
    M, K = A.shape
    N = B.shape[0]
    C = np.zeros((M, N), np.float64)
    Cabs = np.zeros((M, N), np.float64)
    _check(lib().oracle_gemm(_p(A), _p(sA), _p(B), _p(sB), M, N, K, _p(C), _p(Cabs)), "gemm")
    return C, Cabs


def gemm_sampled(A, sA, B, sB, mi, ni):
    M, K = A.shape
    N = B.shape[0]
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    C = np.zeros(len(mi), np.float64)
    Cabs = np.zeros(len(mi), np.float64)
    _check(lib().oracle_gemm_sampled(_p(A), _p(sA), _p(B), _p(sB), M, N, K, _p(mi), _p(ni),
                                     len(mi), _p(C), _p(Cabs)), "gemm_sampled")
    return C, Cabs


def grouped_gemm_ragged_m(A, sA, B, sB, group_end):
    """A [T][K], B [G][N][K] -> C [T][N] (rows outside every group stay 0)."""
    T, K = A.shape
    G, N, _ = B.shape
    ge = np.ascontiguousarray(group_end, dtype=np.int32)
    C = np.zeros((T, N), np.float64)
    Cabs = np.zeros((T, N), np.float64)
    _check(lib().oracle_grouped_gemm_ragged_m(_p(A), _p(sA), _p(B), _p(sB), T, N, K, _p(ge), G,
                                              _p(C), _p(Cabs)), "grouped_gemm_ragged_m")
    return C, Cabs


def grouped_gemm_ragged_m_sampled(A, sA, B, sB, group_end, mi, ni):
    T, K = A.shape
    G, N, _ = B.shape
    ge = np.ascontiguousarray(group_end, dtype=np.int32)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    C = np.zeros(len(mi), np.float64)
    Cabs = np.zeros(len(mi), np.float64)
    _check(lib().oracle_grouped_gemm_ragged_m_sampled(
        _p(A), _p(sA), _p(B), _p(sB), T, N, K, _p(ge), G, _p(mi), _p(ni), len(mi),
        _p(C), _p(Cabs)), "grouped_gemm_ragged_m_sampled")
    return C, Cabs


def grouped_gemm_ragged_k(A, sA, B, sB, group_end):
    """A [M][ldk], B [N][ldk] grouped token-axis copies -> C [G][M][N]."""
    M, ldk = A.shape
    N = B.shape[0]
    ge = np.ascontiguousarray(group_end, dtype=np.int32)
    G = len(ge)
    C = np.zeros((G, M, N), np.float64)
    Cabs = np.zeros((G, M, N), np.float64)
    _check(lib().oracle_grouped_gemm_ragged_k(_p(A), _p(sA), _p(B), _p(sB), M, N, ldk, _p(ge), G,
                                              _p(C), _p(Cabs)), "grouped_gemm_ragged_k")
    return C, Cabs


def grouped_gemm_ragged_k_sampled(A, sA, B, sB, group_end, gi, mi, ni):
    M, ldk = A.shape
    N = B.shape[0]
    ge = np.ascontiguousarray(group_end, dtype=np.int32)
    gi = np.ascontiguousarray(gi, dtype=np.int32)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    C = np.zeros(len(mi), np.float64)
    Cabs = np.zeros(len(mi), np.float64)
    _check(lib().oracle_grouped_gemm_ragged_k_sampled(
        _p(A), _p(sA), _p(B), _p(sB), M, N, ldk, _p(ge), len(ge), _p(gi), _p(mi), _p(ni),
        len(mi), _p(C), _p(Cabs)), "grouped_gemm_ragged_k_sampled")
    return C, Cabs
