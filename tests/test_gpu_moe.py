"""GPU parity of the grouped (MoE expert) GEMMs: ragged M (forward, input
gradient) and ragged K (per-expert weight gradient), the grouped token-axis
quantisation feeding it, and the dual-axis vs forward/backward-split
schedules (which must give bitwise identical gradients).

Every GEMM output is held to |err| <= 1e-5 * sum|ab|.  Experts with at most
1024 tokens reduce with one real product per 8-product MFMA group (exact group
sums); the full-size tests check every output of the MoE layer's three
GEMMs, on the Zipf(1.1)-weight routing and on the Zipf-law routing."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_bytes_equal, assert_gemm_close, bits, deq, host, mxq, scaled_randn, unpack_scales)
from moe_grouped_gemm_mxq_amd import workloads

pytestmark = pytest.mark.gpu

SIZES = [[5, 0, 33, 1, 257, 64], [0, 0, 300], [300, 0, 0], [1], [0, 31, 0, 32, 0, 33, 512, 0],
         [513, 4, 1024, 0, 1500]]


def ragged_m_case(sizes, K, N, seed, lo=-6, hi=6):
    m = mxq()
    T, G = sum(sizes), len(sizes)
    X = scaled_randn((T + 5, K), seed, lo=lo, hi=hi)           # 5 trailing rows in no group
    W = scaled_randn((G * K, N), seed + 1, lo=lo, hi=hi, axis=1).reshape(G, K, N)
    ge = np.cumsum(sizes).astype(np.int32)
    qx = m.quantize(X.cuda(), 1)
    qw = m.quantize_batched(W.cuda(), 2)                        # B[g] = column copy of W[g]
    C = torch.full((T + 5, N), 3.0, device="cuda")
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_M, qx["q_row"], qx["s_row"], qw["q_colT"], qw["s_colT"], C,
                       torch.from_numpy(ge).cuda())
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_row(bits(X))
    refB = [oracle.mxfp8_quant_colT(bits(W[g])) for g in range(G)]
    Bq = np.stack([b[0] for b in refB])
    Bs = np.stack([b[1] for b in refB])
    Cr, Ca = oracle.grouped_gemm_ragged_m(A, sA, Bq, Bs, ge)
    return host(C), Cr, Ca, T


@pytest.mark.parametrize("sizes", SIZES)
def test_ragged_m_small(sizes):
    got, Cr, Ca, T = ragged_m_case(sizes, 160, 72, sum(sizes))
    assert_gemm_close(got[:T], Cr[:T], Ca[:T], f"ragged M {sizes} K 160")
    assert np.all(got[T:] == 3.0)                            # rows in no group untouched


@pytest.mark.parametrize("K", [1056, 2048])
def test_ragged_m_plain_path(K):
    """K above 1024: the plain MFMA loop, groups with partial and 128-row
    aligned tiles."""
    sizes = [5, 0, 133, 1, 257, 300]
    got, Cr, Ca, T = ragged_m_case(sizes, K, 264, K)
    assert_gemm_close(got[:T], Cr[:T], Ca[:T], f"ragged M {sizes} K {K}")
    assert np.all(got[T:] == 3.0)


def ragged_k_case(sizes, Mh, N, seed, axis=1, lo=-6, hi=6):
    m = mxq()
    X = scaled_randn((sum(sizes), Mh), seed, lo=lo, hi=hi, axis=axis)
    dY = scaled_randn((sum(sizes), N), seed + 1, lo=lo, hi=hi, axis=axis)
    ge_np = np.cumsum(sizes).astype(np.int32)
    ge = torch.from_numpy(ge_np).cuda()
    qx = m.quantize_grouped(X.cuda(), ge, 2)
    qy = m.quantize_grouped(dY.cuda(), ge, 2, ldq=qx["ldq"])
    C = m.grouped_gemm(m.MXQ_GG_RAGGED_K, qx["q_colT"], qx["s_colT"], qy["q_colT"], qy["s_colT"], ge)
    torch.cuda.synchronize()
    ldq = qx["ldq"]
    A, sA = oracle.mxfp8_quant_grouped_colT(bits(X), ge_np, ldq)
    B, sB = oracle.mxfp8_quant_grouped_colT(bits(dY), ge_np, ldq)
    Cr, Ca = oracle.grouped_gemm_ragged_k(A, sA, B, sB, ge_np)
    return host(C), Cr, Ca


@pytest.mark.parametrize("sizes", SIZES)
def test_ragged_k_small(sizes):
    got, Cr, Ca = ragged_k_case(sizes, 70, 90, sum(sizes) + 2)
    assert_gemm_close(got, Cr, Ca, f"ragged K {sizes}")
    for g, s in enumerate(sizes):
        if s == 0:
            assert np.all(got[g] == 0.0), f"empty group {g} not exactly zero"


def test_ragged_k_exact_groups_on_spread_tokens():
    """Experts of at most 1024 tokens reduce with exact 8-product groups: with
    every token scaled by its own power of two (2^-8 .. 2^7, so each 32-token
    block spans 2^15), only fp32 accumulation error remains."""
    sizes = [5, 0, 33, 1, 257, 64, 512, 1024, 100]
    got, Cr, Ca = ragged_k_case(sizes, 72, 40, 91, axis=0, lo=-8, hi=8)
    ratio = assert_gemm_close(got, Cr, Ca, f"ragged K {sizes}, spread tokens")
    assert ratio < 0.2 * 1e-5


# ------------------------------------------------------------------ malformed group ends
@pytest.mark.parametrize("ends", [[2 ** 31 - 1, 0, 100], [0, 2 ** 31 - 1, 7, 2 ** 31 - 1, 40],
                                  [-5, 70, 30, 2 ** 31 - 1]])
def test_malformed_group_end_stays_in_bounds(ends):
    """Group ends that are not non-decreasing or lie past T break the
    precondition (results are unspecified) but are clamped on the device:
    the grouped quantisers (MXFP8 and MXFP4) and the grouped GEMMs (E4M3
    ragged M and K, E2M1 ragged K) finish without touching
    memory outside their buffers (guard bytes around the outputs stay), and
    the validator reports the first bad entry."""
    m = mxq()
    T, C, N = 96, 64, 48
    ge = torch.tensor(ends, dtype=torch.int32, device="cuda")
    G = len(ends)
    x = scaled_randn((T, C), 5).cuda()
    ldq = m.mxq_grouped_cols_max(T, G)
    guard = 4096

    def guarded(shape, dtype, fill):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * guard,), fill, dtype=dtype, device="cuda")
        return buf, buf[guard:guard + n].view(shape)

    qbuf, q = guarded((C, ldq), torch.uint8, 0x5A)
    sbuf, s = guarded(m.scale_shape(C, ldq // 32), torch.uint8, 0x5A)
    m.mxq_quantize_grouped(x, ge, ldq, m.MXQ_AXIS_COLT, q_colT=q, s_colT=s)
    # weight gradient over the token-axis copy (B: zero codes, unit scales)
    qy = torch.zeros((N, ldq), dtype=torch.uint8, device="cuda")
    sy = torch.full(m.scale_shape(N, ldq // 32), 127, dtype=torch.uint8, device="cuda")
    cbuf, dW = guarded((G, C, N), torch.float32, 7.0)
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_K, q, s, qy, sy, dW, ge)
    # expert forward over the row copy
    xr = m.quantize(x, m.MXQ_AXIS_ROW)
    wq = torch.zeros((G, N, C), dtype=torch.uint8, device="cuda")
    ws = torch.full((G,) + m.scale_shape(N, C // 32), 127, dtype=torch.uint8, device="cuda")
    ybuf, Y = guarded((T, N), torch.float32, 7.0)
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_M, xr["q_row"], xr["s_row"], wq, ws, Y, ge)
    # MXFP4: grouped token-axis quantiser of fp32 input and the E2M1 weight gradient
    q4buf, q4 = guarded((C, ldq // 2), torch.uint8, 0x5A)
    s4buf, s4 = guarded(m.scale_shape(C, ldq // 32), torch.uint8, 0x5A)
    m.mxq_quantize_fp4_grouped(x.float(), ge, ldq, q4, s4)
    qy4 = torch.zeros((N, ldq // 2), dtype=torch.uint8, device="cuda")
    c4buf, dW4 = guarded((G, C, N), torch.float32, 7.0)
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_K, q4, s4, qy4, sy, dW4, ge, fmt=m.MXQ_FMT_E2M1)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.mxq_validate_group_end(ge, T, flag)
    torch.cuda.synchronize()
    for buf, fill in ((qbuf, 0x5A), (sbuf, 0x5A), (cbuf, 7.0), (ybuf, 7.0), (q4buf, 0x5A), (s4buf, 0x5A),
                      (c4buf, 7.0)):
        assert bool((buf[:guard] == fill).all()) and bool((buf[-guard:] == fill).all()), "guard bytes overwritten"
    bad = next(i for i, e in enumerate(ends) if e < (ends[i - 1] if i else 0) or e < 0 or e > T)
    assert int(flag.item()) == bad + 1


# ------------------------------------------------------------------ full size
def moe_layer_on_gpu(routing):
    """The MoE expert layer on the GPU, dual-axis schedule: 131072 routed
    rows, 32 experts, 7168 -> 4096."""
    m = mxq()
    X, W, dY, ge = workloads.moe_layer(device="cuda", routing=routing)
    ge = ge.cuda()
    G, K, N = W.shape
    # forward: X by rows; W[g] on both axes in one read
    qx = m.quantize(X, 1)
    qw = {"q_row": torch.empty((G * K, N), dtype=torch.uint8, device="cuda"),
          "s_row": torch.empty(m.scale_shape(G * K, N // 32), dtype=torch.uint8, device="cuda"),
          "q_colT": torch.empty((G, N, K), dtype=torch.uint8, device="cuda"),
          "s_colT": torch.empty((G,) + m.scale_shape(N, K // 32), dtype=torch.uint8, device="cuda")}
    for g in range(G):   # K % 32 == 0: expert g's rows are row groups [g*K/32, (g+1)*K/32)
        m.mxq_quantize(W[g], 3, qw["q_row"][g * K:(g + 1) * K], qw["s_row"][g * K // 128:(g + 1) * K // 128],
                       qw["q_colT"][g], qw["s_colT"][g])
    Y = m.grouped_gemm(m.MXQ_GG_RAGGED_M, qx["q_row"], qx["s_row"], qw["q_colT"], qw["s_colT"], ge)
    # backward: dY by rows and grouped token axis in one read; X grouped token axis
    qy = m.quantize_grouped(dY, ge, 3)
    qxt = m.quantize_grouped(X, ge, 2, ldq=qy["ldq"])
    dX = m.grouped_gemm(m.MXQ_GG_RAGGED_M, qy["q_row"], qy["s_row"],
                        qw["q_row"].view(G, K, N), qw["s_row"].view(G, K // 128, N // 32, 32, 4), ge)
    dW = m.grouped_gemm(m.MXQ_GG_RAGGED_K, qxt["q_colT"], qxt["s_colT"], qy["q_colT"], qy["s_colT"], ge)
    torch.cuda.synchronize()
    return dict(X=X, W=W, dY=dY, ge=ge, ge_np=host(ge), qx=qx, qw=qw, qy=qy, qxt=qxt, Y=Y, dX=dX, dW=dW)


@pytest.fixture(scope="module")
def moe_full():
    return moe_layer_on_gpu("zipf_weights")


@pytest.fixture(scope="module")
def moe_weights_ref(moe_full):
    """The oracle's copies of the expert weights (shared by both routings:
    W does not depend on the routing): W[g] along K (forward B[g] = [N][K])
    and along N (input-gradient B[g] = [K][N])."""
    W = moe_full["W"]
    colT, row = [], []
    for g in range(W.shape[0]):
        b = bits(W[g])
        colT.append(oracle.mxfp8_quant_colT(b))
        row.append(oracle.mxfp8_quant_row(b))
    return dict(colT=colT, row=row)


def activations_ref(layer):
    """The oracle's row and grouped token-axis copies of X and dY."""
    ge_np, ldq = layer["ge_np"], layer["qy"]["ldq"]
    ref = {}
    for name, key in (("x", "X"), ("y", "dY")):
        b = bits(layer[key])
        ref[name + "_row"] = oracle.mxfp8_quant_row(b)
        ref[name + "_tok"] = oracle.mxfp8_quant_grouped_colT(b, ge_np, ldq)
        del b
    return ref


@pytest.fixture(scope="module")
def moe_act_ref(moe_full):
    return activations_ref(moe_full)


def group_spans(ge_np):
    start = 0
    for g, e in enumerate(np.asarray(ge_np).tolist()):
        yield g, start, e
        start = e


def check_quantised_copies(layer, act, wref):
    P = oracle.grouped_cols(layer["ge_np"])
    T = layer["X"].shape[0]
    for name, q, key in (("x", layer["qx"], "x_row"), ("y", layer["qy"], "y_row")):
        assert_bytes_equal(host(q["q_row"]), act[key][0], f"{name} row codes")
        assert_bytes_equal(unpack_scales(q["s_row"], T), act[key][1], f"{name} row scales")
    for name, q, key in (("x", layer["qxt"], "x_tok"), ("y", layer["qy"], "y_tok")):
        rq, rs = act[key]
        assert_bytes_equal(host(q["q_colT"])[:, :P], rq[:, :P], f"{name} token-axis codes")
        assert_bytes_equal(unpack_scales(q["s_colT"], rq.shape[0])[:, :P // 32], rs[:, :P // 32],
                           f"{name} token-axis scales")
    if wref is not None:
        qw = layer["qw"]
        G, K, N = layer["W"].shape
        srow = unpack_scales(qw["s_row"], G * K)
        for g in range(G):
            assert_bytes_equal(host(qw["q_colT"][g]), wref["colT"][g][0], f"W[{g}] colT codes")
            assert_bytes_equal(unpack_scales(qw["s_colT"][g], N), wref["colT"][g][1], f"W[{g}] colT scales")
            assert_bytes_equal(host(qw["q_row"][g * K:(g + 1) * K]), wref["row"][g][0], f"W[{g}] row codes")
            assert_bytes_equal(srow[g * K:(g + 1) * K], wref["row"][g][1], f"W[{g}] row scales")


def check_ragged_m(layer, act, wref, which, rows_of=None):
    """Outputs of the forward (Y = X W[g]) or input gradient (dX = dY W[g]^T)
    per expert against the oracle's fp64 product of its own codes; all rows
    of every group unless rows_of(g, start, end) picks some."""
    out = host(layer["Y" if which == "fwd" else "dX"])
    aq, as_ = act["x_row" if which == "fwd" else "y_row"]
    worst = 0.0
    for g, s, e in group_spans(layer["ge_np"]):
        if e <= s:
            continue
        rows = np.arange(s, e) if rows_of is None else rows_of(g, s, e)
        b = deq(*(wref["colT"][g] if which == "fwd" else wref["row"][g]))
        Cr, Ca = oracle.gemm_dequantised(deq(aq[rows], as_[rows]), b)
        worst = max(worst, assert_gemm_close(out[rows], Cr, Ca, f"moe {which} expert {g} ({e - s} rows)"))
    return worst


def check_wgrad(layer, act):
    """Every output of every expert's weight gradient; empty experts exact zeros."""
    dW = host(layer["dW"])
    xq, xs = act["x_tok"]
    yq, ys = act["y_tok"]
    P = 0
    for g, s, e in group_spans(layer["ge_np"]):
        w = oracle.ceil32(e - s)
        if w == 0:
            assert not dW[g].any(), f"empty expert {g} has nonzero dW"
            continue
        a = deq(xq[:, P:P + w], xs[:, P // 32:(P + w) // 32])
        b = deq(yq[:, P:P + w], ys[:, P // 32:(P + w) // 32])
        Cr, Ca = oracle.gemm_dequantised(a, b)
        path = "exact groups" if e - s <= 1024 else "plain"
        assert_gemm_close(dW[g], Cr, Ca, f"moe wgrad expert {g} ({e - s} tokens, {path})")
        P += w


def test_moe_routing_matches_frozen_sizes(moe_full):
    sizes = np.diff(np.concatenate([[0], moe_full["ge_np"]]))
    assert sizes.tolist() == workloads.moe_group_sizes()
    assert (sizes == 0).sum() == 11 and (sizes % 32 != 0).sum() == 16


def test_moe_full_quantised_copies_exact(moe_full, moe_act_ref, moe_weights_ref):
    """Every byte of X's row and token-axis copies, dY's row and token-axis
    copies and all 32 experts' weight copies on both axes equals the oracle's."""
    check_quantised_copies(moe_full, moe_act_ref, moe_weights_ref)


@pytest.mark.parametrize("which", ["fwd", "dgrad"])
def test_moe_ragged_m_every_output(moe_full, moe_act_ref, moe_weights_ref, which):
    worst = check_ragged_m(moe_full, moe_act_ref, moe_weights_ref, which)
    print(f"moe {which}: every output, max err/sum|ab| = {worst:.3e}")


def test_moe_wgrad_every_output(moe_full, moe_act_ref):
    check_wgrad(moe_full, moe_act_ref)


def test_moe_gemms_write_every_output_deterministically(moe_full):
    """Every output tile is written exactly as before when the outputs start as
    NaN: the persistent tile walks (ragged M, ragged K largest group first) miss no tile
    and give the same bits on a second run."""
    m = mxq()
    G, K, N = moe_full["W"].shape
    T = moe_full["X"].shape[0]
    qx, qw, qy, qxt, ge = moe_full["qx"], moe_full["qw"], moe_full["qy"], moe_full["qxt"], moe_full["ge"]
    Y = torch.full((T, N), float("nan"), device="cuda")
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_M, qx["q_row"], qx["s_row"], qw["q_colT"], qw["s_colT"], Y, ge)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y).all()) and torch.equal(Y, moe_full["Y"])
    del Y
    dW = torch.full((G, K, N), float("nan"), device="cuda")
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_K, qxt["q_colT"], qxt["s_colT"], qy["q_colT"], qy["s_colT"], dW, ge)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dW).all()) and torch.equal(dW, moe_full["dW"])


def test_moe_batched_expert_quant_equals_per_expert(moe_full):
    """All 32 experts' dual-axis quantisation in one batched launch gives the
    per-expert launches' bytes exactly (those are checked against the oracle
    in test_moe_full_quantised_copies_exact)."""
    m = mxq()
    W = moe_full["W"]
    G, K, N = W.shape
    qb = m.quantize_batched(W, 3)
    torch.cuda.synchronize()
    qw = moe_full["qw"]
    assert torch.equal(qb["q_row"].view(G * K, N), qw["q_row"])
    assert torch.equal(qb["s_row"].view(qw["s_row"].shape), qw["s_row"])
    assert torch.equal(qb["q_colT"], qw["q_colT"])
    assert torch.equal(qb["s_colT"], qw["s_colT"])


def test_moe_fb_split_equals_dual(moe_full):
    """fb-split: the forward quantises W[g] on its reduction axis only and the
    backward re-quantises it along N; the gradients must equal the dual-axis
    schedule's bit for bit."""
    m = mxq()
    W, ge, G = moe_full["W"], moe_full["ge"], moe_full["W"].shape[0]
    K, N = W.shape[1], W.shape[2]
    fwd_only = m.quantize(W.reshape(G * K, N), 1)  # backward re-quantisation along N (rows of W[g])
    assert torch.equal(fwd_only["q_row"], moe_full["qw"]["q_row"])
    assert torch.equal(fwd_only["s_row"], moe_full["qw"]["s_row"])
    qy = moe_full["qy"]
    dX = m.grouped_gemm(m.MXQ_GG_RAGGED_M, qy["q_row"], qy["s_row"],
                        fwd_only["q_row"].view(G, K, N), fwd_only["s_row"].view(G, K // 128, N // 32, 32, 4), ge)
    torch.cuda.synchronize()
    assert torch.equal(dX, moe_full["dX"])


def test_moe_dual_x_copies_equal_separate_quantisations(moe_full):
    """The dual-axis schedule quantises X by rows and by tokens within each
    expert group from one read in the forward; fb-split quantises it by rows in
    the forward and by tokens in the backward.  Both copies, and the weight
    gradient built on the token-axis copy, must be the same bit for bit."""
    m = mxq()
    X, ge = moe_full["X"], moe_full["ge"]
    both = m.quantize_grouped(X, ge, 3, ldq=moe_full["qy"]["ldq"])
    for k in ("q_row", "s_row"):
        assert torch.equal(both[k], moe_full["qx"][k]), k
    # token-axis copies: the written columns only (each group's tokens padded
    # to 32; the rest of the ceil32(T + 31 G) columns is never written)
    used = oracle.grouped_cols(moe_full["ge_np"])
    assert torch.equal(both["q_colT"][:, :used], moe_full["qxt"]["q_colT"][:, :used])
    assert torch.equal(both["s_colT"][:, :used // 32], moe_full["qxt"]["s_colT"][:, :used // 32])
    qy = moe_full["qy"]
    dW = m.grouped_gemm(m.MXQ_GG_RAGGED_K, both["q_colT"], both["s_colT"], qy["q_colT"], qy["s_colT"], ge)
    torch.cuda.synchronize()
    assert torch.equal(dW, moe_full["dW"])


# ------------------------------------------------------------------ Zipf-law routing
@pytest.fixture(scope="module")
def moe_law(moe_full):
    del moe_full  # (only orders the fixtures: the weight copies are shared)
    return moe_layer_on_gpu("zipf_law")


def test_moe_zipf_law_routing(moe_law, moe_weights_ref):
    """The second routing (expert popularity (e+1)^-1.1: no empty expert, every
    size off a multiple of 32): the activation copies bit-exact, the weight
    gradient of every expert on every output, and the forward and input
    gradient on the first, last and eight random rows of every group (all
    columns)."""
    sizes = np.diff(np.concatenate([[0], moe_law["ge_np"]]))
    assert sizes.tolist() == workloads.moe_group_sizes("zipf_law")
    assert sizes.min() > 0 and (sizes % 32 != 0).all()
    act = activations_ref(moe_law)
    check_quantised_copies(moe_law, act, None)
    rng = np.random.default_rng(17)

    def rows_of(g, s, e):
        return np.unique(np.concatenate([[s, s + 1, e - 2, e - 1], rng.integers(s, e, 8)]))

    for which in ("fwd", "dgrad"):
        check_ragged_m(moe_law, act, moe_weights_ref, which, rows_of)
    check_wgrad(moe_law, act)


# ------------------------------------------------------------------ many groups
def many_group_sizes(G, seed):
    """Mostly empty groups, some of 1-40 rows, three of 257: exercises group
    tables larger than a workgroup, long runs of empty experts and partial
    tiles."""
    rng = np.random.default_rng(seed)
    sizes = np.where(rng.random(G) < 0.85, 0, rng.integers(1, 41, G))
    sizes[rng.choice(G, 3, replace=False)] = 257
    return sizes.astype(np.int64)


@pytest.mark.parametrize("G", [600, 1024])
def test_ragged_m_many_groups(G):
    m = mxq()
    sizes = many_group_sizes(G, G)
    T, K, N = int(sizes.sum()), 64, 40
    X = scaled_randn((T, K), G, lo=-6, hi=6)
    W = scaled_randn((G * K, N), G + 1, lo=-6, hi=6, axis=1).reshape(G, K, N)
    ge = np.cumsum(sizes).astype(np.int32)
    qx = m.quantize(X.cuda(), 1)
    qw = m.quantize_batched(W.cuda(), 2)                     # B[g] = column copy of W[g]
    C = m.grouped_gemm(m.MXQ_GG_RAGGED_M, qx["q_row"], qx["s_row"], qw["q_colT"], qw["s_colT"],
                       torch.from_numpy(ge).cuda())
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_row(bits(X))
    refB = [oracle.mxfp8_quant_colT(bits(W[g])) for g in range(G)]
    Bq = np.stack([b[0] for b in refB])
    Bs = np.stack([b[1] for b in refB])
    Cr, Ca = oracle.grouped_gemm_ragged_m(A, sA, Bq, Bs, ge)
    assert_gemm_close(host(C), Cr, Ca, f"ragged M, {G} groups")


@pytest.mark.parametrize("G", [600, 1024])
def test_ragged_k_many_groups(G):
    sizes = many_group_sizes(G, G + 7)
    got, Cr, Ca = ragged_k_case(sizes.tolist(), 40, 48, G + 2)
    assert_gemm_close(got, Cr, Ca, f"ragged K, {G} groups")
    assert not got[sizes == 0].any(), "empty experts must get exact zeros"
