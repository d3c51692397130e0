"""GPU parity of the grouped (MoE expert) GEMMs: ragged M (forward, input
gradient) and ragged K (per-expert weight gradient), the grouped token-axis
quantisation feeding it, and the dual-axis vs forward/backward-split
schedules (which must give bitwise identical gradients)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_gemm_close, bits, boundary_indices, host, mfma_group_bound, mxq, ragged_k_bound,
                      ragged_m_bound, scale_rows, scaled_randn)
from moe_grouped_gemm_mxq_amd import workloads

pytestmark = pytest.mark.gpu

SIZES = [[5, 0, 33, 1, 257, 64], [0, 0, 300], [300, 0, 0], [1], [0, 31, 0, 32, 0, 33, 512, 0]]


@pytest.mark.parametrize("sizes", SIZES)
def test_ragged_m_small(sizes):
    m = mxq()
    T, K, N, G = sum(sizes), 160, 72, len(sizes)
    X = scaled_randn((T + 5, K), T, lo=-6, hi=6)           # 5 trailing rows in no group
    W = scaled_randn((G * K, N), T + 1, lo=-6, hi=6, axis=1).reshape(G, K, N)
    ge = np.cumsum(sizes).astype(np.int32)
    qx = m.quantize(X.cuda(), 1)
    # B[g] = column copy of W[g] [K][N] -> [N][K]
    qwT = [m.quantize(W[g].cuda(), 2) for g in range(G)]
    B = torch.stack([q["q_colT"] for q in qwT])
    sB = torch.stack([q["s_colT"] for q in qwT])
    C = torch.full((T + 5, N), 3.0, device="cuda")
    m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_M, qx["q_row"], qx["s_row"], B.contiguous(), sB.contiguous(),
                       C, torch.from_numpy(ge).cuda())
    torch.cuda.synchronize()
    A, sA = oracle.mxfp8_quant_row(bits(X))
    refB = [oracle.mxfp8_quant_colT(bits(W[g])) for g in range(G)]
    Bq = np.stack([b[0] for b in refB])
    Bs = np.stack([b[1] for b in refB])
    Cr, Ca = oracle.grouped_gemm_ragged_m(A, sA, Bq, Bs, ge)
    got = host(C)
    hw = ragged_m_bound(A, sA, Bq, Bs, ge)
    assert_gemm_close(got[:T], Cr[:T], Ca[:T], f"ragged M {sizes}", hw_bound=hw[:T])
    assert np.all(got[T:] == 3.0)                            # rows in no group untouched


@pytest.mark.parametrize("sizes", SIZES)
def test_ragged_k_small(sizes):
    m = mxq()
    T, Mh, N, G = sum(sizes), 70, 90, len(sizes)
    X = scaled_randn((T, Mh), T + 2, lo=-6, hi=6, axis=1)
    dY = scaled_randn((T, N), T + 3, lo=-6, hi=6, axis=1)
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
    got = host(C)
    assert_gemm_close(got, Cr, Ca, f"ragged K {sizes}", hw_bound=ragged_k_bound(A, sA, B, sB, ge_np))
    for g, s in enumerate(sizes):
        if s == 0:
            assert np.all(got[g] == 0.0), f"empty group {g} not exactly zero"


# ------------------------------------------------------------------ full size
@pytest.fixture(scope="module")
def moe_full():
    """MoE expert layer, one GPU's 32 experts: 131072 routed rows, 7168 -> 4096,
    Zipf(1.1) top-8 routing (11 empty groups, 16 sizes not multiples of 32)."""
    m = mxq()
    X, W, dY, ge = workloads.moe_layer(device="cuda")
    ge = ge.cuda()
    G, K, N = W.shape
    T = X.shape[0]
    Wflat = W.reshape(G * K, N)
    # forward (dual-axis schedule): X by rows; W[g] on both axes in one read
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
    return dict(X=X, W=W, dY=dY, ge=ge, ge_np=host(ge), qx=qx, qw=qw, qy=qy, qxt=qxt, Y=Y, dX=dX, dW=dW,
                Wflat=Wflat)


def group_rows(ge_np, rng, per_group=6):
    """A few rows of every non-empty group, always including its first and last."""
    rows, start = [], 0
    for e in ge_np.tolist():
        if e > start:
            pick = {start, e - 1} | set(rng.integers(start, e, per_group).tolist())
            rows += sorted(pick)
        start = e
    return np.asarray(rows, np.int64)


def group_of(ge_np, r):
    return int(np.searchsorted(ge_np, r, side="right"))


def test_moe_routing_matches_frozen_sizes(moe_full):
    sizes = np.diff(np.concatenate([[0], moe_full["ge_np"]]))
    assert sizes.tolist() == workloads.moe_group_sizes()
    assert (sizes == 0).sum() == 11 and (sizes % 32 != 0).sum() == 16


@pytest.mark.parametrize("which", ["fwd", "dgrad"])
def test_moe_ragged_m_full_sampled(moe_full, which):
    rng = np.random.default_rng(11 if which == "fwd" else 12)
    ge_np = moe_full["ge_np"]
    rows = group_rows(ge_np, rng)
    if which == "fwd":
        src, out, W = moe_full["X"], moe_full["Y"], moe_full["W"]
        cols = boundary_indices(out.shape[1], 256, rng, 48)
    else:
        src, out, W = moe_full["dY"], moe_full["dX"], moe_full["W"]
        cols = boundary_indices(out.shape[1], 256, rng, 48)
    A, sA = oracle.mxfp8_quant_row(bits(src[torch.as_tensor(rows, device="cuda")]))
    got = host(out[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")])
    worst = 0.0
    for g in sorted({group_of(ge_np, r) for r in rows}):
        sel = np.nonzero([group_of(ge_np, r) == g for r in rows])[0]
        if which == "fwd":   # B[g] = W[g] [K][N] along K, columns `cols`
            B, sB = oracle.mxfp8_quant_row(np.ascontiguousarray(bits(W[g][:, torch.as_tensor(cols, device="cuda")].contiguous()).T))
        else:                # B[g] = W[g] along N, rows `cols`
            B, sB = oracle.mxfp8_quant_row(bits(W[g][torch.as_tensor(cols, device="cuda")]))
        Cr, Ca = oracle.gemm(np.ascontiguousarray(A[sel]), np.ascontiguousarray(sA[sel]), B, sB)
        worst = max(worst, assert_gemm_close(got[sel], Cr, Ca, f"moe {which} group {g}"))
    print(f"moe {which}: {got.size} sampled outputs, max err/sum|ab| = {worst:.3e}")


def test_moe_grouped_token_quant_sampled(moe_full):
    rng = np.random.default_rng(13)
    ge_np = moe_full["ge_np"]
    for name, src in (("qxt", "X"), ("qy", "dY")):
        x = moe_full[src]
        cols = boundary_indices(x.shape[1], 128, rng, 24)
        q = moe_full[name]
        qr, sr = oracle.mxfp8_quant_grouped_colT(bits(x[:, torch.as_tensor(cols, device="cuda")].contiguous()),
                                                 ge_np, q["ldq"])
        P = oracle.grouped_cols(ge_np)
        idx = torch.as_tensor(cols, device="cuda")
        assert np.array_equal(host(q["q_colT"][idx])[:, :P], qr[:, :P]), name
        assert np.array_equal(scale_rows(q["s_colT"], cols)[:, :P // 32], sr[:, :P // 32]), name


def test_moe_wgrad_ragged_k_full_sampled(moe_full):
    rng = np.random.default_rng(14)
    ge_np = moe_full["ge_np"]
    dW = moe_full["dW"]
    G, K, N = dW.shape
    ki = boundary_indices(K, 256, rng, 24)
    ni = boundary_indices(N, 256, rng, 24)
    X, dY = moe_full["X"], moe_full["dY"]
    ldq = moe_full["qy"]["ldq"]
    A, sA = oracle.mxfp8_quant_grouped_colT(bits(X[:, torch.as_tensor(ki, device="cuda")].contiguous()), ge_np, ldq)
    B, sB = oracle.mxfp8_quant_grouped_colT(bits(dY[:, torch.as_tensor(ni, device="cuda")].contiguous()), ge_np, ldq)
    Cr, Ca = oracle.grouped_gemm_ragged_k(A, sA, B, sB, ge_np)
    got = host(dW[:, torch.as_tensor(ki, device="cuda")][:, :, torch.as_tensor(ni, device="cuda")])
    # the reduction runs over one expert's tokens, which can be a handful: the
    # FP8 MFMA group-truncation term is part of the bound (strict ratio reported)
    ratio = assert_gemm_close(got, Cr, Ca, "moe wgrad", hw_bound=ragged_k_bound(A, sA, B, sB, ge_np))
    big = np.diff(np.concatenate([[0], ge_np])) >= 4096
    strict = float(np.max(np.abs(got[big] - Cr[big]) / np.where(Ca[big] > 0, Ca[big], 1)))
    assert strict <= 1e-5, f"experts with >= 4096 tokens: max err/sum|ab| = {strict:.3e}"
    print(f"moe wgrad: {got.size} sampled outputs, max err/sum|ab| = {ratio:.3e} "
          f"(experts with >= 4096 tokens: {strict:.3e})")
    sizes = np.diff(np.concatenate([[0], ge_np]))
    for g in np.nonzero(sizes == 0)[0]:
        assert int(torch.count_nonzero(dW[g]).item()) == 0, f"empty expert {g} has nonzero dW"


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
    in test_moe_ragged_m_full_sampled)."""
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
    sizes = np.diff(np.concatenate([[0], moe_full["ge_np"]]))
    used = int(((sizes + 31) // 32 * 32).sum())
    assert torch.equal(both["q_colT"][:, :used], moe_full["qxt"]["q_colT"][:, :used])
    assert torch.equal(both["s_colT"][:, :used // 32], moe_full["qxt"]["s_colT"][:, :used // 32])
    qy = moe_full["qy"]
    dW = m.grouped_gemm(m.MXQ_GG_RAGGED_K, both["q_colT"], both["s_colT"], qy["q_colT"], qy["s_colT"], ge)
    torch.cuda.synchronize()
    assert torch.equal(dW, moe_full["dW"])


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
    assert_gemm_close(host(C), Cr, Ca, f"ragged M, {G} groups", hw_bound=ragged_m_bound(A, sA, Bq, Bs, ge))


@pytest.mark.parametrize("G", [600, 1024])
def test_ragged_k_many_groups(G):
    m = mxq()
    sizes = many_group_sizes(G, G + 7)
    T, Mh, N = int(sizes.sum()), 40, 48
    X = scaled_randn((T, Mh), G + 2, lo=-6, hi=6, axis=1)
    dY = scaled_randn((T, N), G + 3, lo=-6, hi=6, axis=1)
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
    assert_gemm_close(got, Cr, Ca, f"ragged K, {G} groups", hw_bound=ragged_k_bound(A, sA, B, sB, ge_np))
    assert not got[sizes == 0].any(), "empty experts must get exact zeros"
