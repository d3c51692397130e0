"""ctypes binding of libmxq (include/mxq.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmxq.so``; PyTorch supplies device memory and streams.  Importing
this module fails loudly (RuntimeError) when the library is not built -- there
is no fallback.

Functions named like the C entry points take every buffer from the caller;
the lower-case helpers (``quantize``, ``gemm`` ...) allocate the outputs with
``torch.empty`` and call them.

GEMM operand scale arrays are uint8 tensors of shape ``scale_shape(rows,
nblk)`` = ``(ceil128(rows) // 128, nblk, 32, 4)``: element
``[r // 128, b, r % 32, (r // 32) % 4]`` is the E8M0 scale of row ``r``,
block ``b`` (the layout of include/mxq.h: each dword holds the scales of
rows r, r+32, r+64, r+96 of a 128-row group for one block).
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MXQ_LIB_PATH") or os.path.join(HERE, "libmxq.so")

MXQ_OK = 0
MXQ_ERR_INVALID_ARGUMENT = 1
MXQ_ERR_UNSUPPORTED = 2
MXQ_ERR_DEVICE = 3
MXQ_ERR_LAUNCH = 4
STATUS_NAMES = {0: "MXQ_OK", 1: "MXQ_ERR_INVALID_ARGUMENT", 2: "MXQ_ERR_UNSUPPORTED",
                3: "MXQ_ERR_DEVICE", 4: "MXQ_ERR_LAUNCH"}

MXQ_AXIS_ROW = 1
MXQ_AXIS_COLT = 2
MXQ_FMT_E4M3 = 0
MXQ_FMT_E2M1 = 1
MXQ_GG_RAGGED_M = 0
MXQ_GG_RAGGED_K = 1
BLOCK = 32
MAX_GROUPS = 1024
MAX_ROW_BYTES = 1 << 23  # MXQ_GEMM_MAX_ROW_BYTES: GEMM code rows (K, or K/2 for E2M1) stay below this

EXPORTED = [
    "mxq_abi_version", "mxq_last_error", "mxq_device_check", "mxq_grouped_cols_max", "mxq_operand_sizes",
    "mxq_quantize", "mxq_quantize_batched", "mxq_quantize_grouped", "mxq_qdq_fp4", "mxq_qdq_fp4_ex",
    "mxq_ste_backward_fp4", "mxq_fp4_scale_threshold", "mxq_quantize_fp4", "mxq_gemm", "mxq_grouped_gemm",
    "mxq_validate_group_end", "mxq_quantize_fp4_grouped",
]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise RuntimeError(
            f"libmxq.so not found at {path}. Build it with "
            "`python -m moe_grouped_gemm_mxq_amd.build` (hipcc, gfx950) or point MXQ_LIB_PATH at a build.")
    lib = ctypes.CDLL(path)
    P, I64, I32, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    sig = {
        "mxq_abi_version": ([], I),
        "mxq_last_error": ([], ctypes.c_char_p),
        "mxq_device_check": ([I], I),
        "mxq_grouped_cols_max": ([I64, I32], I64),
        "mxq_operand_sizes": ([I64, I64, I, P, P], I),
        "mxq_quantize": ([P, I64, I64, I64, I, P, P, P, P, P], I),
        "mxq_quantize_batched": ([P, I64, I64, I64, I64, I64, I, P, P, P, P, P], I),
        "mxq_quantize_grouped": ([P, I64, I64, I64, P, I32, I64, I, P, P, P, P, P], I),
        "mxq_qdq_fp4": ([P, P, I64, I64, P, P, P], I),
        "mxq_qdq_fp4_ex": ([P, P, I64, I64, ctypes.c_float, P, P, P, P], I),
        "mxq_ste_backward_fp4": ([P, P, P, I64, I64, P], I),
        "mxq_fp4_scale_threshold": ([ctypes.c_float, P, P], I),
        "mxq_quantize_fp4": ([P, I64, I64, ctypes.c_float, P, P, P], I),
        "mxq_gemm": ([P, P, P, P, P, I64, I64, I64, I64, I, P], I),
        "mxq_grouped_gemm": ([I, P, P, P, P, P, I64, I64, I64, P, I32, I, P], I),
        "mxq_validate_group_end": ([P, I32, I64, P, P], I),
        "mxq_quantize_fp4_grouped": ([P, I64, I64, I64, P, I32, I64, ctypes.c_float, P, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


ABI_VERSION = 7  # MXQ_ABI_VERSION of include/mxq.h this binding is written against

_lib = _load()
if _lib.mxq_abi_version() != ABI_VERSION:
    raise RuntimeError(f"libmxq.so at {LIB_PATH} implements ABI {_lib.mxq_abi_version()}, this binding needs "
                       f"{ABI_VERSION}: rebuild it with `python -m moe_grouped_gemm_mxq_amd.build`")


class MxqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.mxq_last_error().decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def _check(status: int, where: str):
    if status != MXQ_OK:
        raise MxqError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, dtype, name, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")


def ceil32(v: int) -> int:
    return (v + BLOCK - 1) // BLOCK * BLOCK


def scale_shape(rows: int, nblk: int) -> tuple:
    """Shape of the GEMM-operand scale array of `rows` rows and `nblk` blocks per row."""
    return ((rows + 127) // 128, nblk, BLOCK, 4)


def _need_out(t, name, shape):
    if t is None:
        return
    _need(t, torch.uint8, name)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 tensor of shape {tuple(shape)}, got {tuple(t.shape)}")


# ------------------------------------------------------------------ C entry points
def mxq_abi_version() -> int:
    return _lib.mxq_abi_version()


def mxq_last_error() -> str:
    return _lib.mxq_last_error().decode()


def mxq_device_check(device: int = 0) -> int:
    return _lib.mxq_device_check(device)


def mxq_grouped_cols_max(T: int, G: int) -> int:
    return _lib.mxq_grouped_cols_max(T, G)


def mxq_operand_sizes(rows: int, K: int, fmt: int = 0) -> tuple:
    """(code bytes, scale bytes) of a quantised GEMM operand of `rows` rows and reduction length K."""
    c, sc = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.mxq_operand_sizes(rows, K, fmt, ctypes.byref(c), ctypes.byref(sc)), "mxq_operand_sizes")
    return c.value, sc.value


def mxq_quantize(x, axis_mask, q_row=None, s_row=None, q_colT=None, s_colT=None, stream=None):
    """x bf16 [R][C] (unit column stride, any row stride)."""
    _need(x, torch.bfloat16, "x", 2)
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along its last dim")
    R, C = x.shape
    _need_out(q_row, "q_row", (R, ceil32(C)))
    _need_out(s_row, "s_row", scale_shape(R, ceil32(C) // BLOCK))
    _need_out(q_colT, "q_colT", (C, ceil32(R)))
    _need_out(s_colT, "s_colT", scale_shape(C, ceil32(R) // BLOCK))
    _check(_lib.mxq_quantize(_ptr(x), R, C, x.stride(0), axis_mask, _ptr(q_row), _ptr(s_row),
                             _ptr(q_colT), _ptr(s_colT), _stream(stream, x.device)), "mxq_quantize")


def mxq_quantize_batched(x, axis_mask, q_row=None, s_row=None, q_colT=None, s_colT=None, stream=None):
    """x bf16 [batch][R][C] (unit stride along C).  Outputs: q_row [batch][R][Cp],
    s_row (batch,) + scale_shape(R, Cp/32), q_colT [batch][C][Rp], s_colT (batch,) + scale_shape(C, Rp/32)."""
    _need(x, torch.bfloat16, "x", 3)
    if x.stride(2) != 1:
        raise ValueError("x must have unit stride along its last dim")
    nb, R, C = x.shape
    _need_out(q_row, "q_row", (nb, R, ceil32(C)))
    _need_out(s_row, "s_row", (nb,) + scale_shape(R, ceil32(C) // BLOCK))
    _need_out(q_colT, "q_colT", (nb, C, ceil32(R)))
    _need_out(s_colT, "s_colT", (nb,) + scale_shape(C, ceil32(R) // BLOCK))
    _check(_lib.mxq_quantize_batched(_ptr(x), nb, R, C, x.stride(1), x.stride(0), axis_mask, _ptr(q_row),
                                     _ptr(s_row), _ptr(q_colT), _ptr(s_colT), _stream(stream, x.device)),
           "mxq_quantize_batched")


def mxq_quantize_grouped(x, group_end, ldq, axis_mask, q_row=None, s_row=None, q_colT=None,
                         s_colT=None, stream=None):
    _need(x, torch.bfloat16, "x", 2)
    _need(group_end, torch.int32, "group_end", 1)
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along its last dim")
    T, C = x.shape
    _need_out(q_row, "q_row", (T, ceil32(C)))
    _need_out(s_row, "s_row", scale_shape(T, ceil32(C) // BLOCK))
    _need_out(q_colT, "q_colT", (C, ldq))
    _need_out(s_colT, "s_colT", scale_shape(C, ldq // BLOCK))
    _check(_lib.mxq_quantize_grouped(_ptr(x), T, C, x.stride(0), _ptr(group_end), group_end.numel(),
                                     ldq, axis_mask, _ptr(q_row), _ptr(s_row), _ptr(q_colT),
                                     _ptr(s_colT), _stream(stream, x.device)), "mxq_quantize_grouped")


def mxq_qdq_fp4(x, y, codes=None, scales=None, stream=None):
    """x, y fp32 contiguous, same shape; blocks along the last dim."""
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y")
    if not (x.is_contiguous() and y.is_contiguous()) or x.shape != y.shape:
        raise ValueError("x and y must be contiguous and of the same shape")
    L = x.shape[-1] if x.dim() else 1
    rows = x.numel() // L if L else 0
    _check(_lib.mxq_qdq_fp4(_ptr(x), _ptr(y), rows, L, _ptr(codes), _ptr(scales),
                            _stream(stream, x.device)), "mxq_qdq_fp4")


def _rows_L(x):
    L = x.shape[-1] if x.dim() else 1
    return (x.numel() // L if L else 0), L


def _need_u8(t, name, shape):
    if t is None:
        return
    _need(t, torch.uint8, name)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with shape {tuple(shape)}, got {tuple(t.shape)}")


def mxq_qdq_fp4_ex(x, y, scale_factor=6.0, codes=None, scales=None, sat_mask=None, stream=None):
    """As mxq_qdq_fp4 with a runtime scale factor and the optional saturation
    mask uint8 [rows][ceil32(L)/8] (bit j of byte k: element 8k+j clipped)."""
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y")
    if not (x.is_contiguous() and y.is_contiguous()) or x.shape != y.shape:
        raise ValueError("x and y must be contiguous and of the same shape")
    rows, L = _rows_L(x)
    _need_u8(codes, "codes", (rows, ceil32(L) // 2))
    _need_u8(scales, "scales", (rows, ceil32(L) // BLOCK))
    _need_u8(sat_mask, "sat_mask", (rows, ceil32(L) // 8))
    _check(_lib.mxq_qdq_fp4_ex(_ptr(x), _ptr(y), rows, L, float(scale_factor), _ptr(codes), _ptr(scales),
                               _ptr(sat_mask), _stream(stream, x.device)), "mxq_qdq_fp4_ex")


def mxq_ste_backward_fp4(grad_y, sat_mask, grad_x, stream=None):
    """grad_x = 0 where sat_mask marks a clipped element, grad_y elsewhere."""
    _need(grad_y, torch.float32, "grad_y")
    _need(grad_x, torch.float32, "grad_x")
    if not (grad_y.is_contiguous() and grad_x.is_contiguous()) or grad_y.shape != grad_x.shape:
        raise ValueError("grad_y and grad_x must be contiguous and of the same shape")
    rows, L = _rows_L(grad_y)
    _need_u8(sat_mask, "sat_mask", (rows, ceil32(L) // 8))
    _check(_lib.mxq_ste_backward_fp4(_ptr(grad_y), _ptr(sat_mask), _ptr(grad_x), rows, L,
                                     _stream(stream, grad_y.device)), "mxq_ste_backward_fp4")


def mxq_fp4_scale_threshold(scale_factor):
    """Host only: (F, T) of the exponent rule for this scale factor."""
    F, T = ctypes.c_int32(), ctypes.c_uint32()
    _check(_lib.mxq_fp4_scale_threshold(float(scale_factor), ctypes.byref(F), ctypes.byref(T)),
           "mxq_fp4_scale_threshold")
    return F.value, T.value


def _elems(nbytes: int, fmt: int) -> int:
    """K (elements) of an operand row of `nbytes` code bytes."""
    return nbytes * 2 if fmt == MXQ_FMT_E2M1 else nbytes


def mxq_gemm(A, sA, B, sB, C, stream=None, fmt=MXQ_FMT_E4M3):
    """A uint8 [M][K] + scales scale_shape(M, K/32), B [N][K] + scale_shape(N, K/32) -> C fp32 [M][ldc >= N].
    fmt MXQ_FMT_E2M1: A [M][K/2], B [N][K/2] (two E2M1 codes per byte)."""
    for t, n in ((A, "A"), (sA, "sA"), (B, "B"), (sB, "sB")):
        _need(t, torch.uint8, n)
    _need(C, torch.float32, "C", 2)
    M, Kb = A.shape
    K = _elems(Kb, fmt)
    N = B.shape[0]
    if (B.dim() != 2 or B.shape[1] != Kb or tuple(sA.shape) != scale_shape(M, K // BLOCK)
            or tuple(sB.shape) != scale_shape(N, K // BLOCK)):
        raise ValueError("operand shapes disagree")
    if not all(t.is_contiguous() for t in (A, sA, B, sB)):
        raise ValueError("operands must be contiguous")
    if C.shape[0] != M or C.shape[1] < N or C.stride(1) != 1:
        raise ValueError("C must be [M][>=N] with unit column stride")
    _check(_lib.mxq_gemm(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(C), M, N, K, C.stride(0),
                         fmt, _stream(stream, A.device)), "mxq_gemm")


def mxq_grouped_gemm(mode, A, sA, B, sB, C, group_end, stream=None, fmt=MXQ_FMT_E4M3):
    """RAGGED_M: A [M][K], B [G][N][K], C [M][N].  RAGGED_K: A [M][K], B [N][K], C [G][M][N].

    Scales: sA scale_shape(M, K/32); sB (G,) + scale_shape(N, K/32) (ragged M) or scale_shape(N, K/32).
    fmt MXQ_FMT_E2M1: code rows of K/2 bytes (ragged K: from mxq_quantize_fp4_grouped)."""
    for t, n in ((A, "A"), (sA, "sA"), (B, "B"), (sB, "sB")):
        _need(t, torch.uint8, n)
    _need(C, torch.float32, "C")
    _need(group_end, torch.int32, "group_end", 1)
    G = group_end.numel()
    M, Kb = A.shape
    K = _elems(Kb, fmt)
    N = B.shape[-2]
    if mode == MXQ_GG_RAGGED_M:
        ok = (tuple(B.shape) == (G, N, Kb) and tuple(sB.shape) == (G,) + scale_shape(N, K // BLOCK)
              and tuple(C.shape) == (M, N))
    else:
        N = B.shape[0]
        ok = (tuple(B.shape) == (N, Kb) and tuple(sB.shape) == scale_shape(N, K // BLOCK)
              and tuple(C.shape) == (G, M, N))
    if not ok or tuple(sA.shape) != scale_shape(M, K // BLOCK):
        raise ValueError("grouped GEMM operand shapes disagree")
    if not all(t.is_contiguous() for t in (A, sA, B, sB, C)):
        raise ValueError("operands must be contiguous")
    _check(_lib.mxq_grouped_gemm(mode, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(C), M, N, K,
                                 _ptr(group_end), G, fmt, _stream(stream, A.device)),
           "mxq_grouped_gemm")


def mxq_quantize_fp4(x, codes, scales, scale_factor=6.0, stream=None):
    """MXFP4 GEMM operand: x fp32 [rows][L] -> codes uint8 [rows][ceil32(L)/2],
    scales scale_shape(rows, ceil32(L)/32) (the GEMM operand layout)."""
    _need(x, torch.float32, "x")
    if not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous 2-D tensor")
    rows, L = x.shape
    _need_u8(codes, "codes", (rows, ceil32(L) // 2))
    _need_u8(scales, "scales", scale_shape(rows, ceil32(L) // BLOCK))
    _check(_lib.mxq_quantize_fp4(_ptr(x), rows, L, float(scale_factor), _ptr(codes), _ptr(scales),
                                 _stream(stream, x.device)), "mxq_quantize_fp4")


def mxq_quantize_fp4_grouped(x, group_end, ldq, codes, scales, scale_factor=6.0, stream=None):
    """Grouped token-axis MXFP4 operand: x fp32 [T][C] (unit column stride) ->
    codes uint8 [C][ldq/2], scales scale_shape(C, ldq/32) (the operand layout)."""
    _need(x, torch.float32, "x", 2)
    _need(group_end, torch.int32, "group_end", 1)
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along its last dim")
    T, C = x.shape
    _need_u8(codes, "codes", (C, ldq // 2))
    _need_u8(scales, "scales", scale_shape(C, ldq // BLOCK))
    _check(_lib.mxq_quantize_fp4_grouped(_ptr(x), T, C, x.stride(0), _ptr(group_end), group_end.numel(), ldq,
                                         float(scale_factor), _ptr(codes), _ptr(scales), _stream(stream, x.device)),
           "mxq_quantize_fp4_grouped")


def mxq_validate_group_end(group_end, T, flag, stream=None):
    _need(group_end, torch.int32, "group_end", 1)
    _need(flag, torch.int32, "flag")
    _check(_lib.mxq_validate_group_end(_ptr(group_end), group_end.numel(), T, _ptr(flag),
                                       _stream(stream, group_end.device)), "mxq_validate_group_end")


# ------------------------------------------------------------------ allocate-and-call helpers
def _u8(shape, device):
    return torch.empty(shape, dtype=torch.uint8, device=device)


def quantize(x, axis_mask=MXQ_AXIS_ROW | MXQ_AXIS_COLT, stream=None):
    """Returns a dict with 'q_row', 's_row' and/or 'q_colT', 's_colT'."""
    R, C = x.shape
    out = {}
    if axis_mask & MXQ_AXIS_ROW:
        out["q_row"] = _u8((R, ceil32(C)), x.device)
        out["s_row"] = _u8(scale_shape(R, ceil32(C) // BLOCK), x.device)
    if axis_mask & MXQ_AXIS_COLT:
        out["q_colT"] = _u8((C, ceil32(R)), x.device)
        out["s_colT"] = _u8(scale_shape(C, ceil32(R) // BLOCK), x.device)
    mxq_quantize(x, axis_mask, out.get("q_row"), out.get("s_row"), out.get("q_colT"),
                 out.get("s_colT"), stream)
    return out


def quantize_batched(x, axis_mask=MXQ_AXIS_ROW | MXQ_AXIS_COLT, stream=None):
    """x bf16 [batch][R][C] -> dict of batched outputs (see mxq_quantize_batched)."""
    nb, R, C = x.shape
    out = {}
    if axis_mask & MXQ_AXIS_ROW:
        out["q_row"] = _u8((nb, R, ceil32(C)), x.device)
        out["s_row"] = _u8((nb,) + scale_shape(R, ceil32(C) // BLOCK), x.device)
    if axis_mask & MXQ_AXIS_COLT:
        out["q_colT"] = _u8((nb, C, ceil32(R)), x.device)
        out["s_colT"] = _u8((nb,) + scale_shape(C, ceil32(R) // BLOCK), x.device)
    mxq_quantize_batched(x, axis_mask, out.get("q_row"), out.get("s_row"), out.get("q_colT"), out.get("s_colT"),
                         stream)
    return out


def quantize_grouped(x, group_end, axis_mask=MXQ_AXIS_COLT, ldq=None, stream=None):
    T, C = x.shape
    if ldq is None:
        ldq = mxq_grouped_cols_max(T, group_end.numel())
    out = {"ldq": ldq}
    if axis_mask & MXQ_AXIS_ROW:
        out["q_row"] = _u8((T, ceil32(C)), x.device)
        out["s_row"] = _u8(scale_shape(T, ceil32(C) // BLOCK), x.device)
    if axis_mask & MXQ_AXIS_COLT:
        out["q_colT"] = _u8((C, ldq), x.device)
        out["s_colT"] = _u8(scale_shape(C, ldq // BLOCK), x.device)
    mxq_quantize_grouped(x, group_end, ldq, axis_mask, out.get("q_row"), out.get("s_row"),
                         out.get("q_colT"), out.get("s_colT"), stream)
    return out


def qdq_fp4(x, want_codes=False, stream=None):
    y = torch.empty_like(x)
    codes = scales = None
    if want_codes:
        L = x.shape[-1]
        rows = x.numel() // L
        codes = _u8((rows, ceil32(L) // 2), x.device)
        scales = _u8((rows, ceil32(L) // BLOCK), x.device)
    mxq_qdq_fp4(x, y, codes, scales, stream)
    return (y, codes, scales) if want_codes else y


def quantize_fp4(x, scale_factor=6.0, stream=None):
    """MXFP4 GEMM operand of a 2-D fp32 tensor: (codes, scales in the operand layout)."""
    rows, L = x.shape
    codes = _u8((rows, ceil32(L) // 2), x.device)
    scales = _u8(scale_shape(rows, ceil32(L) // BLOCK), x.device)
    mxq_quantize_fp4(x, codes, scales, scale_factor, stream)
    return codes, scales


def quantize_fp4_grouped(x, group_end, ldq=None, scale_factor=6.0, stream=None):
    """Grouped token-axis MXFP4 operand of x fp32 [T][C]: {"ldq", "codes", "scales"}."""
    T, C = x.shape
    if ldq is None:
        ldq = mxq_grouped_cols_max(T, group_end.numel())
    out = {"ldq": ldq, "codes": _u8((C, ldq // 2), x.device), "scales": _u8(scale_shape(C, ldq // BLOCK), x.device)}
    mxq_quantize_fp4_grouped(x, group_end, ldq, out["codes"], out["scales"], scale_factor, stream)
    return out


def qdq_fp4_ste(x, scale_factor=6.0, want_codes=False, stream=None):
    """Forward of the clipped-STE fake quantiser: returns (y, sat_mask) or,
    with want_codes, (y, sat_mask, codes, scales)."""
    rows, L = _rows_L(x)
    y = torch.empty_like(x)
    mask = _u8((rows, ceil32(L) // 8), x.device)
    codes = scales = None
    if want_codes:
        codes = _u8((rows, ceil32(L) // 2), x.device)
        scales = _u8((rows, ceil32(L) // BLOCK), x.device)
    mxq_qdq_fp4_ex(x, y, scale_factor, codes, scales, mask, stream)
    return (y, mask, codes, scales) if want_codes else (y, mask)


def ste_backward_fp4(grad_y, sat_mask, stream=None):
    grad_x = torch.empty_like(grad_y)
    mxq_ste_backward_fp4(grad_y, sat_mask, grad_x, stream)
    return grad_x


def gemm(A, sA, B, sB, stream=None, fmt=MXQ_FMT_E4M3):
    C = torch.empty((A.shape[0], B.shape[0]), dtype=torch.float32, device=A.device)
    mxq_gemm(A, sA, B, sB, C, stream, fmt)
    return C


def grouped_gemm(mode, A, sA, B, sB, group_end, stream=None, fmt=MXQ_FMT_E4M3):
    if mode == MXQ_GG_RAGGED_M:
        C = torch.empty((A.shape[0], B.shape[1]), dtype=torch.float32, device=A.device)
    else:
        C = torch.empty((group_end.numel(), A.shape[0], B.shape[0]), dtype=torch.float32, device=A.device)
    mxq_grouped_gemm(mode, A, sA, B, sB, C, group_end, stream, fmt)
    return C
