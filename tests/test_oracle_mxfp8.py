"""Pins for the oracle's MXFP8 quantisation (row, column, dual, grouped).

What fixes the answer (never the oracle's own formula):
* the E4M3 element format through PyTorch's ``float8_e4m3fn`` (decode of all
  256 codes; round-to-nearest-even encode of every distinct encoder input,
  with the saturating clamp at 448 applied before the cast);
* exact rational brute force on tiny shapes, with the shared exponent found
  by comparing against powers of two rather than by frexp;
* closed forms: the scale byte is the bf16 exponent field of the block
  maximum minus 8, and the maximum element lands in the top binade;
* invariants: quantise(dequantise(q, s)) == (q, s); the column copy of X is
  the row copy of X^T; a grouped copy with one group is the column copy, and
  every group is the column copy of its own rows, zero padded.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_mxq_amd.workloads import bf16_bits


def torch_e4m3(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, np.float32)).clamp(-448, 448)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_value(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def bf16_of(x: torch.Tensor) -> np.ndarray:
    return bf16_bits(x.to(torch.bfloat16))


# ---------------------------------------------------------------- elements
def test_e4m3_decode_all_codes_match_torch():
    ref = torch_e4m3_value(np.arange(256, dtype=np.uint8))
    for c in range(256):
        v = oracle.e4m3_decode(c)
        if c in (0x7F, 0xFF):
            assert np.isnan(v) and np.isnan(ref[c])
        else:
            assert v == ref[c], hex(c)


def test_e4m3_encode_every_distinct_input_matches_torch():
    """Encoder inputs are bf16 values times powers of two: 8-bit significands
    at any exponent.  Every such magnitude from 2^-40 up to 2^10 (below rounds
    to zero, above saturates) plus zero, both signs."""
    m = np.arange(128, 256, dtype=np.float64)
    vals = np.concatenate([(m * 2.0 ** e) for e in range(-47, 3)])     # 2^-40 .. 2^10
    vals = np.concatenate([vals, -vals, [0.0, -0.0]]).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode_array(vals), torch_e4m3(vals))


def test_e4m3_encode_random_fp32_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-600, 600, 200000),
                        rng.standard_normal(200000) * 2.0 ** rng.integers(-14, 9, 200000)])
    v = v.astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode_array(v), torch_e4m3(v))


def test_e4m3_rounding_spot_values():
    enc = oracle.e4m3_encode
    assert enc(464.0) == 0x7E          # tie between 448 and (absent) 480 -> even 448
    assert enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(1.0625) == 0x38         # tie 1.0 / 1.125 -> even mantissa (1.0)
    assert enc(1.1875) == 0x3A         # tie 1.125 / 1.25 -> 1.25 (even)
    assert enc(2.0 ** -10) == 0x00     # half of the smallest subnormal -> 0
    assert enc(-2.0 ** -10) == 0x80
    assert enc(3 * 2.0 ** -11) == 0x02 - 1   # 1.5 * 2^-10 -> 2^-9 (code 1)


# ---------------------------------------------------------------- brute force
def brute_mxfp8_block(vals):
    """Exact-rational block: shared exponent s with 2^(s+8) <= amax < 2^(s+9),
    clamped to [-127, 127] (zero block -> -127); each element the nearest
    finite E4M3 value to v/2^s (magnitudes beyond 448 -> 448), ties to the
    code with an even mantissa bit."""
    fl = [float(v) for v in vals] + [0.0] * (32 - len(vals))
    fr = [Fraction(v) for v in fl]
    amax = max(abs(v) for v in fr)
    if amax == 0:
        s = -127
    else:
        s = -200
        while Fraction(2) ** (s + 9) <= amax:
            s += 1
        s = max(min(s, 127), -127)
    table = [(c, Fraction(float(v))) for c, v in enumerate(torch_e4m3_value(np.arange(0x7F, dtype=np.uint8)))]
    codes = []
    for v, f in zip(fr, fl):
        y = min(abs(v) / Fraction(2) ** s, Fraction(448))
        best = min(table, key=lambda cv: (abs(y - cv[1]), cv[0] & 1))[0]
        codes.append(best | (0x80 if np.signbit(f) else 0))
    return codes, s + 127


def brute_row(xb):
    x = xb.view(np.uint16)
    R, C = x.shape
    f = (x.astype(np.uint32) << 16).view(np.float32)
    Cp = oracle.ceil32(C)
    q = np.zeros((R, Cp), np.uint8)
    sc = np.zeros((R, Cp // 32), np.uint8)
    for r in range(R):
        for b in range(Cp // 32):
            codes, byte = brute_mxfp8_block(f[r, b * 32:(b + 1) * 32])
            q[r, b * 32:(b + 1) * 32] = codes
            sc[r, b] = byte
    return q, sc


@pytest.mark.parametrize("shape", [(1, 1), (1, 32), (2, 33), (33, 2), (3, 17), (65, 65)])
def test_bruteforce_row_and_colT(shape):
    g = torch.Generator().manual_seed(sum(shape))
    x = torch.randn(shape, generator=g) * torch.exp2(torch.randint(-30, 30, shape, generator=g).float())
    xb = bf16_of(x)
    q, s = oracle.mxfp8_quant_row(xb)
    bq, bs = brute_row(xb)
    assert np.array_equal(q, bq) and np.array_equal(s, bs)
    qt, st = oracle.mxfp8_quant_colT(xb)
    bqt, bst = brute_row(np.ascontiguousarray(xb.T))
    assert np.array_equal(qt, bqt) and np.array_equal(st, bst)


def test_bruteforce_extreme_blocks():
    rows = [
        [0.0] * 32,                                         # zero block -> byte 0
        [-0.0, 0.0] * 16,                                   # signed zeros kept
        [2.0 ** -133] + [0.0] * 31,                         # smallest bf16 subnormal
        [3.0e38, -3.0e38] + [1.0] * 30,                     # largest binade
        [2.0 ** -120, 2.0 ** -126, 2.0 ** -130] + [0.0] * 29,   # clamped scale
        [464.0, 448.0, 480.0, 1.0, 1.0625, 1.1875] + [0.0] * 26,
    ]
    xb = bf16_of(torch.tensor(rows, dtype=torch.float32))
    q, s = oracle.mxfp8_quant_row(xb)
    bq, bs = brute_row(xb)
    assert np.array_equal(q, bq) and np.array_equal(s, bs)
    assert s[0, 0] == 0 and np.all(q[1, 0::2] == 0x80) and np.all(q[1, 1::2] == 0)


# ---------------------------------------------------------------- closed forms
def test_scale_byte_is_exponent_field_minus_8():
    g = torch.Generator().manual_seed(11)
    x = torch.randn(64, 256, generator=g) * torch.exp2(torch.randint(-100, 100, (64, 1), generator=g).float())
    xb = bf16_of(x)
    q, s = oracle.mxfp8_quant_row(xb)
    amax_bits = (xb.reshape(64, 8, 32) & 0x7FFF).max(axis=2)
    efield = (amax_bits >> 7).astype(np.int64)
    assert np.array_equal(s.astype(np.int64), np.maximum(efield - 8, 0))
    # the block maximum lands in the top binade [256, 448] (exponent field 15)
    arg = (xb.reshape(64, 8, 32) & 0x7FFF).argmax(axis=2)
    top = np.take_along_axis(q.reshape(64, 8, 32), arg[..., None], axis=2)[..., 0]
    assert np.all((top & 0x78) == 0x78)


def dequant_to_bf16(q, s):
    v = oracle.mxfp8_dequant(q, s)
    return bf16_of(torch.from_numpy(v).to(torch.float32))


def test_quantise_dequantise_is_a_fixed_point():
    g = torch.Generator().manual_seed(12)
    x = torch.randn(40, 96, generator=g) * torch.exp2(torch.randint(-60, 60, (40, 1), generator=g).float())
    q, s = oracle.mxfp8_quant_row(bf16_of(x))
    q2, s2 = oracle.mxfp8_quant_row(dequant_to_bf16(q, s))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ---------------------------------------------------------------- invariants
def test_colT_is_row_copy_of_transpose_and_dual_is_the_pair():
    x = bf16_of(torch.randn(70, 45, generator=torch.Generator().manual_seed(13)))
    qt, st = oracle.mxfp8_quant_colT(x)
    qr, sr = oracle.mxfp8_quant_row(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, qr) and np.array_equal(st, sr)


@pytest.mark.parametrize("sizes", [
    [70], [0, 1, 31, 32, 33, 0], [0, 0, 5], [64, 0], [17, 40, 1, 0, 96],
])
def test_grouped_colT_is_per_group_colT(sizes):
    T = sum(sizes)
    x = bf16_of(torch.randn(T, 40, generator=torch.Generator().manual_seed(len(sizes))))
    ge = np.cumsum(sizes).astype(np.int32)
    ldq = oracle.grouped_cols(ge) + 64          # room past the last group
    q, s = oracle.mxfp8_quant_grouped_colT(x, ge, ldq)
    P, start = 0, 0
    for m in sizes:
        w = oracle.ceil32(m)
        if m:
            qg, sg = oracle.mxfp8_quant_colT(x[start:start + m])
            assert np.array_equal(q[:, P:P + w], qg) and np.array_equal(s[:, P // 32:(P + w) // 32], sg)
            assert np.all(q[:, P + m:P + w] == 0)            # zero-padded tail
        P += w
        start += m
    assert P == oracle.grouped_cols(ge)
    assert np.all(q[:, P:] == 0) and np.all(s[:, P // 32:] == 0)   # untouched
    if len(sizes) == 1:
        qt, st = oracle.mxfp8_quant_colT(x)
        assert np.array_equal(q[:, :P], qt) and np.array_equal(s[:, :P // 32], st)


def test_malformed_group_ends_and_nonfinite_are_rejected():
    x = bf16_of(torch.randn(10, 32))
    with pytest.raises(ValueError):
        oracle.mxfp8_quant_grouped_colT(x, np.array([5, 3], np.int32), 64)
    with pytest.raises(ValueError):
        oracle.mxfp8_quant_grouped_colT(x, np.array([11], np.int32), 64)
    bad = x.copy()
    bad[3, 4] = 0x7FC0                       # NaN
    with pytest.raises(ValueError):
        oracle.mxfp8_quant_row(bad)
