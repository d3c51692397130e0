"""GPU parity of the quantisers (MXFP4 QDQ, MXFP8 row / column / dual /
grouped) against the CPU oracle: codes, scales and dequantised values must be
bit-exact.  The oracle always quantises the seeded bf16/fp32 inputs itself."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bytes_equal, bits, host, mxq, out_host, scaled_randn, unpack_scales
from moe_grouped_gemm_mxq_amd import workloads

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ MXFP4 QDQ
def check_qdq(x: torch.Tensor, what: str):
    m = mxq()
    y, codes, scales = m.qdq_fp4(x.cuda(), want_codes=True)
    torch.cuda.synchronize()
    yr, cr, sr = oracle.mxfp4_qdq(x.numpy(), want_codes=True)
    assert np.array_equal(host(y).view(np.uint32), yr.view(np.uint32)), f"{what}: values differ"
    assert np.array_equal(host(codes), cr), f"{what}: nibbles differ"
    assert np.array_equal(host(scales), sr), f"{what}: scales differ"


def test_qdq_page_test_shapes():
    for x in workloads.qdq_small():
        check_qdq(x, f"qdq {tuple(x.shape)}")


@pytest.mark.parametrize("shape", [(1, 1), (5, 32), (7, 64), (3, 100), (9, 31), (2, 4097)])
def test_qdq_ragged_and_aligned_shapes(shape):
    g = torch.Generator().manual_seed(sum(shape))
    x = torch.randn(shape, generator=g) * torch.exp2(torch.randint(-40, 40, (shape[0], 1), generator=g).float())
    check_qdq(x, f"qdq {shape}")


def test_qdq_crafted_thresholds_ties_and_extremes():
    rows = []
    for E in range(-100, 127, 3):     # the round-half threshold pair in many binades
        for mant in (0x7C3B6, 0x7C3B7):
            a = np.array([(E + 127) << 23 | mant], np.uint32).view(np.float32)[0]
            rows.append([a] + [a * f for f in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.041)] + [0.0] * 23)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for k in (-30, -10, 0, 20, 100):
        s = 2.0 ** k
        rows.append([6 * s] + [m * s for m in mids] + [-m * s for m in mids] + [-0.0, 0.0] * 8 + [1e-45])
    fmax = float(np.finfo(np.float32).max)
    rows.append([fmax, -fmax] + [1.0] * 30)
    rows.append([1e-40, -1e-38] + [0.0] * 30)
    check_qdq(torch.tensor(rows, dtype=torch.float32), "crafted")


def test_qdq_full_size_8192x8192_one_percent_rows_scaled():
    x = workloads.qdq_large()
    check_qdq(x, "qdq 8192x8192")


# ------------------------------------------ MXFP4 with a scale factor, clipped STE
FACTORS = [6.0, 5.0, 7.25, 1.0, 0.75, 12.0, 3.0]


def check_qdq_ex(x: torch.Tensor, sf: float, what: str, xdev=None):
    """GPU y, codes, scales and saturation mask vs the oracle, bit for bit."""
    m = mxq()
    xd = x.cuda() if xdev is None else xdev
    y, mask, codes, scales = m.qdq_fp4_ste(xd, sf, want_codes=True)
    torch.cuda.synchronize()
    yr, cr, sr, mr = oracle.mxfp4_qdq_ex(x.numpy(), sf)
    assert np.array_equal(host(y).view(np.uint32), yr.view(np.uint32)), f"{what} sf={sf}: values differ"
    assert np.array_equal(host(codes), cr), f"{what} sf={sf}: nibbles differ"
    assert np.array_equal(host(scales), sr), f"{what} sf={sf}: scales differ"
    assert np.array_equal(host(mask), mr), f"{what} sf={sf}: saturation masks differ"
    return mask, mr


@pytest.mark.parametrize("sf", FACTORS)
@pytest.mark.parametrize("shape", [(1, 1), (5, 32), (3, 100), (9, 31), (64, 256), (2, 4097)])
def test_qdq_scale_factor_and_mask_bitexact(shape, sf):
    g = torch.Generator().manual_seed(sum(shape) + int(sf * 4))
    x = torch.randn(shape, generator=g) * torch.exp2(torch.randint(-30, 30, (shape[0], 1), generator=g).float())
    check_qdq_ex(x, sf, f"qdq_ex {shape}")


@pytest.mark.parametrize("sf", FACTORS)
def test_qdq_scale_factor_threshold_neighbours(sf):
    """Block maxima at the fp32 neighbours (+-3 ulps) of sf*sqrt(2)*2^n, where
    the exponent steps, in many binades."""
    rows = []
    for n in range(-28, 100, 7):
        a0 = np.float32(np.float32(sf) * np.sqrt(2.0) * 2.0 ** n)
        a = a0
        for _ in range(3):
            a = np.nextafter(a, np.float32(0))
        for _ in range(7):
            rows.append([a] + [a * f for f in (0.04, 0.13, 0.2, 0.37, 0.55, 0.71, -0.9)] + [0.0] * 24)
            a = np.nextafter(a, np.float32(np.inf))
    check_qdq_ex(torch.tensor(np.array(rows, np.float32)), sf, "thresholds")


def test_qdq_scale_factor_unaligned_input_takes_general_path():
    """x and y 4 bytes past a 16-byte boundary with L % 32 == 0: the general
    (per-row) kernel must give the same bits."""
    g = torch.Generator().manual_seed(3)
    x = torch.randn(17 * 64, generator=g) * 3
    base = torch.empty(17 * 64 + 1, device="cuda")
    base[1:] = x.cuda()
    check_qdq_ex(x.view(17, 64), 7.25, "unaligned", xdev=base[1:].view(17, 64))


def test_qdq_ex_at_six_equals_plain_qdq():
    m = mxq()
    x = workloads.qdq_small()[0].cuda()
    y0, c0, s0 = m.qdq_fp4(x, want_codes=True)
    y1, _, c1, s1 = m.qdq_fp4_ste(x, 6.0, want_codes=True)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)) and torch.equal(c0, c1) and torch.equal(s0, s1)


@pytest.mark.parametrize("shape", [(6, 45), (8, 64), (3, 4097), (1, 1)])
@pytest.mark.parametrize("inplace", [False, True])
def test_ste_backward_matches_oracle(shape, inplace):
    m = mxq()
    g = torch.Generator().manual_seed(shape[1])
    x = torch.randn(shape, generator=g)
    x[:, ::7] *= 4.0
    gy = torch.randn(shape, generator=g)
    mask, mr = check_qdq_ex(x, 8.0, f"ste fwd {shape}")
    gyd = gy.cuda()
    if inplace:
        m.mxq_ste_backward_fp4(gyd, mask, gyd)
        gx = gyd
    else:
        gx = m.ste_backward_fp4(gyd, mask)
    torch.cuda.synchronize()
    want = oracle.mxfp4_ste_backward(gy.numpy(), mr)
    assert np.array_equal(host(gx).view(np.uint32), want.view(np.uint32))


def test_ste_full_size_8192x8192():
    """The QDQ workload at full size with the mask, then the masked backward."""
    m = mxq()
    x = workloads.qdq_large()
    mask, mr = check_qdq_ex(x, 6.0, "qdq_ex 8192x8192")
    gy = torch.randn(x.shape, generator=torch.Generator().manual_seed(1))
    gx = m.ste_backward_fp4(gy.cuda(), mask)
    torch.cuda.synchronize()
    want = oracle.mxfp4_ste_backward(gy.numpy(), mr)
    assert np.array_equal(host(gx).view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------------ MXFP8
SHAPES = [(1, 1), (1, 32), (2, 33), (33, 2), (3, 17), (65, 65), (128, 128), (127, 129),
          (300, 257), (256, 1000), (1000, 264), (4097, 40)]


def quant_ref(xb: np.ndarray, axis_mask: int):
    out = {}
    if axis_mask & 1:
        out["q_row"], out["s_row"] = oracle.mxfp8_quant_row(xb)
    if axis_mask & 2:
        out["q_colT"], out["s_colT"] = oracle.mxfp8_quant_colT(xb)
    return out


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("axis", [1, 2, 3])
def test_quantize_bitexact(shape, axis):
    m = mxq()
    x = scaled_randn(shape, seed=shape[0] * 7 + shape[1], zero_rows=min(2, shape[0] // 8))
    got = m.quantize(x.cuda(), axis)
    torch.cuda.synchronize()
    ref = quant_ref(bits(x), axis)
    for k, v in ref.items():
        assert_bytes_equal(out_host(got, k, v.shape[0]), v, f"{k} {shape}")


@pytest.mark.parametrize("R,C", [(300, 257), (97, 8200), (1, 40), (4097, 7168)])
@pytest.mark.parametrize("axis", [1, 2, 3])
def test_quantize_leaves_scale_padding_untouched(R, C, axis):
    """Scale arrays have ceil128(rows) rows; the bytes of rows past `rows` (a
    sentinel here) are never written, by the row kernel or the tile kernel."""
    m = mxq()
    x = scaled_randn((R, C), seed=R + C)
    Cp, Rp = (C + 31) // 32 * 32, (R + 31) // 32 * 32
    dev = torch.device("cuda")
    out = dict(q_row=torch.empty(R, Cp, dtype=torch.uint8, device=dev),
               s_row=torch.full(m.scale_shape(R, Cp // 32), 0xA5, dtype=torch.uint8, device=dev),
               q_colT=torch.empty(C, Rp, dtype=torch.uint8, device=dev),
               s_colT=torch.full(m.scale_shape(C, Rp // 32), 0xA5, dtype=torch.uint8, device=dev))
    row, col = axis & 1, axis & 2
    m.mxq_quantize(x.cuda(), axis, out["q_row"] if row else None, out["s_row"] if row else None,
                   out["q_colT"] if col else None, out["s_colT"] if col else None)
    torch.cuda.synchronize()
    for k, v in quant_ref(bits(x), axis).items():
        if k.startswith("s_"):
            sc = out[k]
            full = host(sc.permute(0, 3, 2, 1).reshape(sc.shape[0] * 128, sc.shape[1]))
            assert np.all(full[v.shape[0]:] == 0xA5), f"{k} padding written {R}x{C}"
            assert_bytes_equal(full[:v.shape[0]], v, f"{k} {R}x{C}")
        else:
            assert_bytes_equal(host(out[k]), v, f"{k} {R}x{C}")


@pytest.mark.parametrize("C,pad", [(200, 8), (203, 3)])
def test_quantize_strided_input(C, pad):
    """x is a column slice of a wider matrix (row stride C+pad)."""
    m = mxq()
    big = scaled_randn((150, C + pad), seed=C)
    x = big.cuda()[:, :C]
    got = m.quantize(x, 3)
    torch.cuda.synchronize()
    ref = quant_ref(bits(big[:, :C].contiguous()), 3)
    for k, v in ref.items():
        assert np.array_equal(out_host(got, k, v.shape[0]), v), k


def test_quantize_extreme_values():
    rows = [[0.0] * 64, [-0.0, 0.0] * 32, [2.0 ** -133] + [0.0] * 63,
            [3.0e38, -3.0e38] + [1.0] * 62, [2.0 ** -120, 2.0 ** -126, 2.0 ** -130] + [0.0] * 61,
            [464.0, 448.0, 480.0, 1.0, 1.0625, 1.1875, -500.0] + [0.0] * 57]
    x = torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    got = mxq().quantize(x.cuda(), 3)
    torch.cuda.synchronize()
    for k, v in quant_ref(bits(x), 3).items():
        assert np.array_equal(out_host(got, k, v.shape[0]), v), k


def exhaustive_blocks():
    """Every (bf16 value, scale byte) pair the quantiser can meet: for each
    scale byte b a pilot of exponent field b+8 fixes the block scale, and the
    other 31 slots of the blocks run through every bf16 pattern (both signs)
    with exponent field <= b+8."""
    blocks = []
    for b in range(0, 247):
        ef = b + 8
        pilot = (ef << 7) | 0x7F
        mags = np.arange(0, (ef + 1) << 7, dtype=np.uint32)     # all patterns with Efield <= ef
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        n = -(-len(vals) // 31)
        vals = np.concatenate([vals, np.zeros(n * 31 - len(vals), np.uint16)]).reshape(n, 31)
        blk = np.concatenate([np.full((n, 1), pilot, np.uint16), vals], axis=1)
        blocks.append(blk)
    return np.concatenate(blocks)


def test_quantize_every_element_and_scale_pair():
    xb = exhaustive_blocks()                              # [n][32] bf16 bits, one block per row
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16)
    m = mxq()
    got = m.quantize(x.cuda(), 1)
    torch.cuda.synchronize()
    q, s = oracle.mxfp8_quant_row(xb)
    assert np.array_equal(unpack_scales(got["s_row"], len(s)), s)
    assert np.array_equal(host(got["q_row"]), q)
    # the same blocks through the column path (blocks running down columns)
    xt = np.ascontiguousarray(xb[:4096].T)                # [32][4096]
    got = m.quantize(torch.from_numpy(xt.view(np.int16)).view(torch.bfloat16).cuda(), 2)
    torch.cuda.synchronize()
    qt, st = oracle.mxfp8_quant_colT(xt)
    assert np.array_equal(host(got["q_colT"]), qt) and np.array_equal(unpack_scales(got["s_colT"], len(st)), st)


@pytest.mark.parametrize("R,C,pad", [(70, 45, 0), (64, 128, 3), (33, 300, 1), (256, 96, 0)])
@pytest.mark.parametrize("axis", [1, 2, 3])
def test_quantize_batched_bitexact(R, C, pad, axis):
    """Three matrices, each padded by `pad` rows in the stacked input (so the
    batch stride exceeds one matrix); every output equals the oracle's."""
    m = mxq()
    nb = 3
    big = scaled_randn((nb * (R + pad), C), seed=R * 3 + C + pad, zero_rows=2)
    x3 = big.view(nb, R + pad, C)[:, :R, :]
    xg = big.cuda().view(nb, R + pad, C)[:, :R, :]   # strided batch view on the device
    assert xg.stride(0) == (R + pad) * C
    got = m.quantize_batched(xg, axis)
    torch.cuda.synchronize()
    for b in range(nb):
        ref = quant_ref(bits(x3[b].contiguous()), axis)
        for k, v in ref.items():
            g = got[k][b]
            h = unpack_scales(g, v.shape[0]) if k.startswith("s_") else host(g)
            assert_bytes_equal(h, v, f"{k} batch {b} {R}x{C}")


GROUPS = [[70], [0, 1, 31, 32, 33, 0], [0, 0, 5], [64, 0], [17, 40, 1, 0, 96],
          [0, 0, 0, 200, 0, 0], [129, 1, 255, 0, 2, 64, 33],
          # 1024 groups (the maximum), mostly empty: tables larger than a workgroup
          np.where(np.random.default_rng(1).random(1024) < 0.85, 0,
                   np.random.default_rng(2).integers(1, 41, 1024)).tolist()]


@pytest.mark.parametrize("sizes", GROUPS)
# one or two column tiles; six (a second column group of two, the last with a
# 40-column tail); nine with odd rows (the unaligned load path, three groups)
@pytest.mark.parametrize("C", [40, 129, 680, 1031])
@pytest.mark.parametrize("axis", [2, 3])
def test_grouped_quantize_bitexact(sizes, C, axis):
    m = mxq()
    T = sum(sizes)
    x = scaled_randn((T, C), seed=T + C)
    ge = np.cumsum(sizes).astype(np.int32)
    got = m.quantize_grouped(x.cuda(), torch.from_numpy(ge).cuda(), axis)
    torch.cuda.synchronize()
    P = oracle.grouped_cols(ge)
    q, s = oracle.mxfp8_quant_grouped_colT(bits(x), ge, got["ldq"])
    assert np.array_equal(host(got["q_colT"])[:, :P], q[:, :P])
    assert np.array_equal(unpack_scales(got["s_colT"], C)[:, :P // 32], s[:, :P // 32])
    if axis & 1:
        qr, sr = oracle.mxfp8_quant_row(bits(x))
        assert np.array_equal(host(got["q_row"]), qr) and np.array_equal(unpack_scales(got["s_row"], T), sr)


def test_validate_group_end():
    m = mxq()
    flag = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    cases = [([0, 3, 3, 10], 10, 0), ([0, 3, 2, 10], 10, 3), ([5, 11], 10, 2), ([-1, 4], 10, 1),
             ([10] * 32, 10, 0)]
    for ge, T, want in cases:
        m.mxq_validate_group_end(torch.tensor(ge, dtype=torch.int32, device="cuda"), T, flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == want, (ge, T)
