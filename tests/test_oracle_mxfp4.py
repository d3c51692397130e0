"""Pins for the oracle's MXFP4 quant-dequant.

What fixes the answer here (never the oracle's own formula):
* the numbers the AMCT FakeQuant page prints in section 2 (tests/golden);
* exact rational arithmetic (``fractions``) with a 60-digit ``decimal``
  logarithm, brute force on the page's test shapes;
* the library routine the page names as equivalent for element rounding
  (``torch.bucketize(y_abs, midpoints, right=True)``);
* closed forms: codebook reproduction, the round-half threshold of the
  exponent, midpoint ties, scaling by powers of two, per-row padding.
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_numeric_model.txt")


def golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, *v = line.split()
                vals[k] = v
    return vals


def e2m1_decode(nib: int) -> float:
    """OCP E2M1: sign | 2 exponent bits (bias 1) | 1 mantissa bit."""
    s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
    v = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
    return -v if s else v


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def qdq_scales(x):
    y, codes, scales = oracle.mxfp4_qdq(np.asarray(x, np.float32), want_codes=True)
    return y, codes, scales.astype(np.int32) - 127


# ---------------------------------------------------------------- golden values
def test_golden_numeric_model_is_consistent():
    g = golden()
    assert int(g["block_size"][0]) == oracle.BLOCK == 32
    cb = [float(v) for v in g["codebook"]]
    # the codebook is exactly the set of non-negative E2M1 values
    assert sorted({abs(e2m1_decode(n)) for n in range(16)}) == cb
    # the midpoints are the means of neighbouring codebook values
    mids = [float(v) for v in g["midpoints"]]
    assert mids == [(a + b) / 2 for a, b in zip(cb, cb[1:])]
    # the printed literal is 2^-30 to its 10 significant digits
    assert float(g["min_scale_raw_literal"][0]) == pytest.approx(2.0 ** -30, rel=1e-9)
    assert int(g["min_scale_raw_log2"][0]) == -30
    assert float(g["scale_factor"][0]) == 6.0 == max(cb)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("k", [-29, -7, -1, 0, 1, 5, 40, 120])
def test_codebook_values_reproduce_exactly(k):
    """amax = 6*2^k gives scale 2^k, and every c*2^k then maps to itself."""
    cb = [float(v) for v in golden()["codebook"]]
    row = [6.0 * 2.0 ** k] + [s * c * 2.0 ** k for c in cb for s in (1, -1)]
    row += [0.0] * (32 - len(row))
    y, _, e = qdq_scales(np.array([row]))
    assert e[0, 0] == k
    assert np.array_equal(bits(y[0]), bits(row))


@pytest.mark.parametrize("k", [-20, 0, 3, 60])
def test_midpoint_ties_go_to_larger_magnitude(k):
    g = golden()
    cb = [float(v) for v in g["codebook"]]
    mids = [float(v) for v in g["midpoints"]]
    s = 2.0 ** k
    at = [m * s for m in mids]
    below = [float(np.nextafter(np.float32(m * s), np.float32(0))) for m in mids]
    row = np.array([[6 * s] + at + [-v for v in at] + below + [0.0] * (32 - 1 - 21)], np.float32)
    y, _, e = qdq_scales(row)
    assert e[0, 0] == k
    assert list(y[0, 1:8]) == [c * s for c in cb[1:]]            # ties round up
    assert list(y[0, 8:15]) == [-c * s for c in cb[1:]]
    assert list(y[0, 15:22]) == [c * s for c in cb[:-1]]        # just below stays down


def test_exponent_round_half_threshold():
    """round(log2(amax/6)) switches between the fp32 neighbours 0x4107C3B6 and
    0x4107C3B7 (3*2^(E+1/2) lies between them), in every binade."""
    for E in range(-100, 127):
        for mant, up in ((0x7C3B6, 0), (0x7C3B7, 1)):
            a = np.array([(E + 127) << 23 | mant], np.uint32).view(np.float32)
            _, _, e = qdq_scales(np.concatenate([a, np.zeros(31, np.float32)])[None])
            want = max(E - 3 + up, -30)
            assert e[0, 0] == want, (E, hex(mant))
    # and the 60-digit logarithm agrees on the pair itself
    getcontext().prec = 60
    for b, want in ((0x4107C3B6, 0), (0x4107C3B7, 1)):
        a = float(np.array([b], np.uint32).view(np.float32)[0])
        L = (Decimal(a) / 6).ln() / Decimal(2).ln()
        assert abs(L - want) < Decimal("0.5")


def dec_round_log2(frac: Fraction) -> int:
    getcontext().prec = 60
    L = (Decimal(frac.numerator).ln() - Decimal(frac.denominator).ln()) / Decimal(2).ln()
    lo = math.floor(L)
    return lo if (L - lo) < (lo + 1 - L) else lo + 1


def test_scale_exponent_matches_high_precision_log2():
    rng = np.random.default_rng(1)
    amax = np.concatenate([
        rng.uniform(0.5, 1.5, 300) * 2.0 ** rng.integers(-140, 127, 300),
        [6 * 2.0 ** -30, 6 * 2.0 ** -30.5, 6 * 2.0 ** -29.5, 1e-40, 2.0 ** -126, 1.0, 6.0, 3e38],
    ]).astype(np.float32)
    for a in amax:
        _, _, e = qdq_scales(np.concatenate([[a], np.zeros(31, np.float32)])[None])
        raw = max(Fraction(float(a)) / 6, Fraction(1, 2 ** 30))
        assert e[0, 0] == dec_round_log2(raw), float(a)


def test_zero_and_tiny_blocks_use_minimum_scale():
    x = np.zeros((1, 64), np.float32)
    x[0, 1] = -0.0
    x[0, 32:] = 1e-12                       # amax/6 < 2^-30: clamped
    x[0, 33] = -0.25 * 2.0 ** -30           # a midpoint of the clamped scale
    y, _, e = qdq_scales(x)
    assert list(e[0]) == [-30, -30]
    assert np.array_equal(bits(y[0, :32]), bits(x[0, :32]))    # zeros, signs kept
    assert y[0, 33] == -0.5 * 2.0 ** -30
    assert np.all(y[0, 34:] == 0.0)


def test_saturation_and_sign_of_zero():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 8.4   # amax: scale 2^0 (8.4 < 6*sqrt2), so 8.4 -> 6 (saturates)
    x[0, 1] = -5.0  # midpoint between 4 and 6 -> -6
    x[0, 2] = -0.1  # rounds to zero, keeps its sign
    y, _, e = qdq_scales(x)
    assert e[0, 0] == 0
    assert y[0, 0] == 6.0 and y[0, 1] == -6.0
    assert y[0, 2] == 0.0 and math.copysign(1, y[0, 2]) == -1


@pytest.mark.parametrize("j", [-17, -3, 4, 25])
def test_power_of_two_scaling_commutes(j):
    x = torch.randn(16, 96, generator=torch.Generator().manual_seed(3)).numpy()
    y = oracle.mxfp4_qdq(x)
    y2 = oracle.mxfp4_qdq((x * 2.0 ** j).astype(np.float32))
    assert np.array_equal(bits(y2), bits(y * np.float32(2.0 ** j)))


def test_rows_are_padded_separately():
    """Each row of a (2,33) input is its own pair of blocks; flattening first
    would put row 1's first 31 values in row 0's second block."""
    x = np.zeros((2, 33), np.float32)
    x[0, :32] = 0.3
    x[0, 32] = 0.01
    x[1, :] = 100.0
    y = oracle.mxfp4_qdq(x)
    for r in range(2):
        assert np.array_equal(bits(y[r]), bits(oracle.mxfp4_qdq(x[r:r + 1])[0]))
    flat = np.concatenate([x.reshape(-1), np.zeros(96 - 66, np.float32)])
    y_flat = oracle.mxfp4_qdq(flat[None])[0][:66].reshape(2, 33)
    assert not np.array_equal(bits(y), bits(y_flat))
    assert y[0, 32] != 0.0 and y_flat[0, 32] == 0.0


# ---------------------------------------------------------------- brute force
def brute_qdq(x: np.ndarray) -> np.ndarray:
    """Exact-rational QDQ of an array (last dim blocked, rows padded alone)."""
    cb = [Fraction(c) for c in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    rows = x.reshape(-1, x.shape[-1])
    L = rows.shape[1]
    out = np.zeros_like(rows)
    for r, row in enumerate(rows):
        for b0 in range(0, L, 32):
            blk = [Fraction(float(v)) for v in row[b0:b0 + 32]]
            amax = max(abs(v) for v in blk)
            e = -30 if amax == 0 else dec_round_log2(max(amax / 6, Fraction(1, 2 ** 30)))
            sc = Fraction(2) ** e
            for i, v in enumerate(blk):
                y = abs(v) / sc
                best = min(cb, key=lambda c: (abs(y - c), -c))      # tie -> larger
                out[r, b0 + i] = math.copysign(float(best * sc), float(row[b0 + i]))
    return out.reshape(x.shape)


def crafted_rows():
    rng = np.random.default_rng(7)
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows.append(np.array([6.0] + mids + [-m for m in mids] + [0.0, -0.0] * 8 + [3.0, -2.5], np.float32))
    rows.append((rng.standard_normal(33) * 2.0 ** 20).astype(np.float32))
    rows.append((rng.standard_normal(33) * 2.0 ** -20).astype(np.float32))
    rows.append(np.array([1e-12] * 16 + [-3e-11] * 17, np.float32))
    rows.append(np.array([8.485281] * 3 + [8.4852819] * 30, np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("case", ["2x33", "3x17", "4x48x33", "crafted"])
def test_bruteforce_exact_rational(case):
    if case == "crafted":
        x = crafted_rows()
    else:
        shapes = {"2x33": (2, 33), "3x17": (3, 17), "4x48x33": (4, 48, 33)}
        x = torch.randn(shapes[case], generator=torch.Generator().manual_seed(0)).numpy()
        x[..., 0] *= 2.0 ** np.arange(x[..., 0].size).reshape(x[..., 0].shape) % 7  # vary scales
    y = oracle.mxfp4_qdq(x)
    assert np.array_equal(bits(y), bits(brute_qdq(x)))


# ---------------------------------------------------------------- library routine
def test_element_rounding_equals_bucketize_right():
    """The page's second implementation rounds with
    bucketize(y_abs, midpoints, right=True); the oracle's codes must agree."""
    x = torch.randn(64, 256, generator=torch.Generator().manual_seed(5)).numpy()
    x[:, ::5] = np.round(x[:, ::5] * 4) / 4          # plant exact midpoints
    y, codes, e = qdq_scales(x)
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.50, 3.50, 5.00], dtype=torch.float64)
    scale = np.repeat(2.0 ** e.astype(np.float64), 32, axis=1)
    yabs = torch.tensor(np.abs(x.astype(np.float64)) / scale)
    idx = torch.bucketize(yabs, mids, right=True).numpy()
    nib = np.zeros_like(idx)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    assert np.array_equal(nib & 7, idx)
    assert np.array_equal(nib >> 3, np.signbit(x).astype(np.int64))
    # nibble decoded as OCP E2M1 times the block scale is the dequantised value
    dec = np.vectorize(e2m1_decode)(nib) * scale
    assert np.array_equal(dec.astype(np.float32), y)


def test_out_of_contract_inputs_are_rejected():
    with pytest.raises(ValueError):
        oracle.mxfp4_qdq(np.array([[np.nan] + [0.0] * 31], np.float32))
    with pytest.raises(ValueError):
        oracle.mxfp4_qdq(np.array([[np.inf] + [0.0] * 31], np.float32))


def test_largest_finite_input_stays_finite():
    """FLT_MAX/6 < 2^125.5, so the exponent never exceeds 125 and 6*2^125 fits."""
    fmax = np.finfo(np.float32).max
    y, _, e = qdq_scales(np.array([[fmax, -fmax] + [1.0] * 30], np.float32))
    assert e[0, 0] == 125
    assert y[0, 0] == 6 * 2.0 ** 125 and y[0, 1] == -6 * 2.0 ** 125


# ---------------------------------------------------------------- runtime scale factor
# The op takes scale_factor (default 6) and divides amax by it before the
# logarithm (AMCT FakeQuant article, section 2 parameters and section 3.3,
# where the op's inv_scale_factor_scale is 6 / scale_factor).
FACTORS = [6.0, 5.0, 7.25, 1.0, 0.75, 4.0, 12.0]


def brute_qdq_sf(x: np.ndarray, sf: float):
    """Exact-rational QDQ with scale factor sf: returns y and the saturation mask
    as booleans (|x| > 6 * scale), both [rows][L]."""
    cb = [Fraction(c) for c in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    rows = x.reshape(-1, x.shape[-1])
    L = rows.shape[1]
    out = np.zeros_like(rows)
    sat = np.zeros(rows.shape, bool)
    fsf = Fraction(float(np.float32(sf)))
    for r, row in enumerate(rows):
        for b0 in range(0, L, 32):
            blk = [Fraction(float(v)) for v in row[b0:b0 + 32]]
            amax = max(abs(v) for v in blk)
            e = -30 if amax == 0 else dec_round_log2(max(amax / fsf, Fraction(1, 2 ** 30)))
            e = max(e, -30)
            sc = Fraction(2) ** e
            for i, v in enumerate(blk):
                y = abs(v) / sc
                best = min(cb, key=lambda c: (abs(y - c), -c))
                out[r, b0 + i] = math.copysign(float(best * sc), float(row[b0 + i]))
                sat[r, b0 + i] = abs(v) > 6 * sc
    return out.reshape(x.shape), sat


def unpack_mask(mask: np.ndarray, L: int) -> np.ndarray:
    return np.unpackbits(mask, axis=1, bitorder="little")[:, :L].astype(bool)


def test_default_factor_equals_plain_qdq():
    x = torch.randn(9, 100, generator=torch.Generator().manual_seed(11)).numpy()
    y0, c0, s0 = oracle.mxfp4_qdq(x, want_codes=True)
    y, c, s, _ = oracle.mxfp4_qdq_ex(x, 6.0)
    assert np.array_equal(bits(y), bits(y0)) and np.array_equal(c, c0) and np.array_equal(s, s0)


@pytest.mark.parametrize("sf", FACTORS)
def test_scale_factor_bruteforce_exact_rational(sf):
    x = torch.randn(3, 70, generator=torch.Generator().manual_seed(int(sf * 8))).numpy()
    x[1] *= 2.0 ** 17
    x[2, :40] *= 2.0 ** -9
    y, _, _, mask = oracle.mxfp4_qdq_ex(x, sf)
    want_y, want_sat = brute_qdq_sf(x, sf)
    assert np.array_equal(bits(y), bits(want_y))
    assert np.array_equal(unpack_mask(mask, 70), want_sat)


def test_scale_factor_threshold_for_several_factors():
    """round(log2(amax/sf)) steps from n to n+1 where amax crosses sf*sqrt(2)*2^n,
    i.e. where amax^2 >= 2*sf^2*4^n.  The fp32 neighbours straddling that point
    are found with exact rationals and must get scale bytes n+127 and n+128."""
    for sf in [5.0, 7.25, 1.0, 0.75, 3.0, 6.0, 10.5]:
        fsf = Fraction(float(np.float32(sf)))
        for n in (-20, -3, 0, 1, 4, 30):
            t2 = 2 * fsf * fsf * Fraction(4) ** n if n >= 0 else 2 * fsf * fsf / Fraction(4) ** -n
            a = np.float32(float(np.float32(sf)) * math.sqrt(2.0) * 2.0 ** n)
            while Fraction(float(a)) ** 2 >= t2:
                a = np.nextafter(a, np.float32(0))
            while Fraction(float(a)) ** 2 < t2:
                a = np.nextafter(a, np.float32(np.inf))
            below = np.nextafter(a, np.float32(0))
            for v, want in ((below, n), (a, n + 1)):
                x = np.zeros((1, 32), np.float32)
                x[0, 5] = v
                _, _, s, _ = oracle.mxfp4_qdq_ex(x, sf)
                assert int(s[0, 0]) - 127 == max(want, -30), (sf, n, float(v))


@pytest.mark.parametrize("j", [-3, -1, 1, 2, 5])
def test_scale_byte_shifts_with_power_of_two_factor(j):
    """Multiplying sf by 2^j divides amax/sf by 2^j: every unclamped scale byte
    drops by exactly j."""
    x = (torch.randn(16, 64, generator=torch.Generator().manual_seed(3)) * 100).numpy()
    _, _, s0, _ = oracle.mxfp4_qdq_ex(x, 5.0)
    _, _, s1, _ = oracle.mxfp4_qdq_ex(x, 5.0 * 2.0 ** j)
    assert np.all(s0.astype(int) - 127 > -20)
    assert np.array_equal(s1.astype(int), s0.astype(int) - j)


def test_saturation_mask_marks_values_beyond_six_scales():
    """sf = 6 and amax = 8: log2(8/6) = 0.415 rounds to 0, scale 1, so 6 is the
    largest code and is reached without clipping; anything above 6 clipped."""
    six_up = float(np.nextafter(np.float32(6), np.float32(7)))
    vals = [8.0, 6.0, six_up, -7.0, 5.99, 0.0, -6.0, 6.5, 5.0, -0.0] + [1.0] * 22
    x = np.array([vals], np.float32)
    y, _, s, mask = oracle.mxfp4_qdq_ex(x, 6.0)
    assert s[0, 0] == 127
    want = np.array([abs(v) > 6.0 for v in vals])
    assert np.array_equal(unpack_mask(mask, 32)[0], want)
    assert y[0, 0] == 6.0 and y[0, 2] == 6.0 and y[0, 3] == -6.0 and y[0, 1] == 6.0
    # on random data with several factors the mask is exactly |x| > 6 * scale
    for sf in (6.0, 4.0, 9.0):
        x = torch.randn(5, 77, generator=torch.Generator().manual_seed(2)).numpy()
        _, _, s, mask = oracle.mxfp4_qdq_ex(x, sf)
        scale = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)[:, :77]
        assert np.array_equal(unpack_mask(mask, 77), np.abs(x.astype(np.float64)) > 6 * scale)
        # padding bits past L stay clear
        assert not np.unpackbits(mask, axis=1, bitorder="little")[:, 77:].any()
    # sf <= 6 never clips: amax / scale < sf * sqrt(2) <= 6 * sqrt(2) only above 6
    x = torch.randn(8, 64, generator=torch.Generator().manual_seed(4)).numpy()
    assert not oracle.mxfp4_qdq_ex(x, 4.0)[3].any()


def test_ste_backward_zeroes_only_clipped_elements():
    """Clipped STE (AMCT FakeQuant article, section 4.1): the gradient passes
    through where the quantiser did not clip and is 0 where it did."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 45)).astype(np.float32)
    x[:, ::7] *= 4.0                                      # make some blocks clip
    g = rng.standard_normal((6, 45)).astype(np.float32)
    _, _, s, mask = oracle.mxfp4_qdq_ex(x, 8.0)
    gx = oracle.mxfp4_ste_backward(g, mask)
    scale = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)[:, :45]
    clipped = np.abs(x.astype(np.float64)) > 6 * scale
    assert clipped.any() and not clipped.all()
    assert np.array_equal(gx, np.where(clipped, np.float32(0), g))
    # an all-clear mask is the identity; an all-set mask gives zeros
    ones = np.full_like(mask, 0xFF)
    assert np.array_equal(oracle.mxfp4_ste_backward(g, np.zeros_like(mask)), g)
    assert not oracle.mxfp4_ste_backward(g, ones).any()


def test_scale_factor_out_of_contract_is_rejected():
    x = np.ones((1, 32), np.float32)
    for sf in (0.0, -6.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            oracle.mxfp4_qdq_ex(x, sf)
    # a block scale above 2^127 is not an E8M0 value
    big = np.full((1, 32), np.finfo(np.float32).max, np.float32)
    with pytest.raises(ValueError):
        oracle.mxfp4_qdq_ex(big, 0.5)
    oracle.mxfp4_qdq_ex(big, 6.0)
