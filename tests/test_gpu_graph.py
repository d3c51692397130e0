"""The hot path recorded into a HIP graph and replayed.

No entry point allocates, synchronises, clears memory with a memset or copies
anything to the host (the group sizes stay on the device), so a training step
built from the library's calls can be captured once (torch.cuda.CUDAGraph,
which records the HIP work enqueued on the capturing stream) and replayed.
Every replay runs after eager work that zeroes every output buffer and calls
the library outside the graph, and must reproduce the eager step bit for bit:
the quantised bytes, the GEMM outputs and the MXFP4 quant-dequant."""
import numpy as np
import pytest
import torch

from gpu_util import mxq, scaled_randn

pytestmark = pytest.mark.gpu


def _u8(*shape):
    return torch.zeros(*shape, dtype=torch.uint8, device="cuda")


def _f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32, device="cuda")


def _dual_bufs(m, R, C):
    """row and colT copies of an R x C bf16 matrix"""
    return {"q_row": _u8(R, m.ceil32(C)), "s_row": _u8(*m.scale_shape(R, m.ceil32(C) // 32)),
            "q_colT": _u8(C, m.ceil32(R)), "s_colT": _u8(*m.scale_shape(C, m.ceil32(R) // 32))}


def test_captured_step_replays_to_the_eager_results():
    m = mxq()
    # dense linear: X [M][K], W [K][N], dY [M][N]
    M, K, N = 384, 640, 320
    X, W, dY = (scaled_randn(s, seed).cuda() for s, seed in (((M, K), 1), ((K, N), 2), ((M, N), 3)))
    # MoE layer: routed rows in expert order, experts W[g] [H][F]
    sizes = [700, 0, 1100, 248]
    T, G, H, F = sum(sizes), len(sizes), 512, 384
    Xm, dYm = scaled_randn((T, H), 4).cuda(), scaled_randn((T, F), 5).cuda()
    Wm = scaled_randn((G * H, F), 6, axis=1).reshape(G, H, F).cuda()
    ge = torch.from_numpy(np.cumsum(sizes).astype(np.int32)).cuda()
    ldq = m.mxq_grouped_cols_max(T, G)
    x4 = (torch.randn(256, 1024, generator=torch.Generator().manual_seed(7)) * 3).cuda()

    o = {}
    o["x"], o["w"], o["dy"] = _dual_bufs(m, M, K), _dual_bufs(m, K, N), _dual_bufs(m, M, N)
    o["y"], o["dx"], o["dw"] = _f32(M, N), _f32(M, K), _f32(K, N)
    o["xm"] = {"q_row": _u8(T, H), "s_row": _u8(*m.scale_shape(T, H // 32))}
    o["wm"] = {"q_row": _u8(G, H, F), "s_row": _u8(G, *m.scale_shape(H, F // 32)),
               "q_colT": _u8(G, F, H), "s_colT": _u8(G, *m.scale_shape(F, H // 32))}
    o["dym"] = {"q_row": _u8(T, F), "s_row": _u8(*m.scale_shape(T, F // 32)),
                "q_colT": _u8(F, ldq), "s_colT": _u8(*m.scale_shape(F, ldq // 32))}
    o["xg"] = {"q_colT": _u8(H, ldq), "s_colT": _u8(*m.scale_shape(H, ldq // 32))}
    o["ym"], o["dxm"], o["dwm"] = _f32(T, F), _f32(T, H), _f32(G, H, F)
    o["fp4"] = {"y": torch.zeros_like(x4), "codes": _u8(256, 512), "scales": _u8(256, 32)}

    def step():
        d = o
        m.mxq_qdq_fp4(x4, d["fp4"]["y"], d["fp4"]["codes"], d["fp4"]["scales"])
        for t, k in ((X, "x"), (W, "w")):
            m.mxq_quantize(t, 3, d[k]["q_row"], d[k]["s_row"], d[k]["q_colT"], d[k]["s_colT"])
        m.mxq_gemm(d["x"]["q_row"], d["x"]["s_row"], d["w"]["q_colT"], d["w"]["s_colT"], d["y"])
        m.mxq_quantize(dY, 3, d["dy"]["q_row"], d["dy"]["s_row"], d["dy"]["q_colT"], d["dy"]["s_colT"])
        m.mxq_gemm(d["dy"]["q_row"], d["dy"]["s_row"], d["w"]["q_row"], d["w"]["s_row"], d["dx"])
        m.mxq_gemm(d["x"]["q_colT"], d["x"]["s_colT"], d["dy"]["q_colT"], d["dy"]["s_colT"], d["dw"])
        m.mxq_quantize(Xm, 1, d["xm"]["q_row"], d["xm"]["s_row"])
        m.mxq_quantize_batched(Wm, 3, d["wm"]["q_row"], d["wm"]["s_row"], d["wm"]["q_colT"], d["wm"]["s_colT"])
        m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_M, d["xm"]["q_row"], d["xm"]["s_row"], d["wm"]["q_colT"],
                           d["wm"]["s_colT"], d["ym"], ge)
        m.mxq_quantize_grouped(dYm, ge, ldq, 3, d["dym"]["q_row"], d["dym"]["s_row"], d["dym"]["q_colT"],
                               d["dym"]["s_colT"])
        m.mxq_quantize_grouped(Xm, ge, ldq, 2, None, None, d["xg"]["q_colT"], d["xg"]["s_colT"])
        m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_M, d["dym"]["q_row"], d["dym"]["s_row"], d["wm"]["q_row"],
                           d["wm"]["s_row"], d["dxm"], ge)
        m.mxq_grouped_gemm(m.MXQ_GG_RAGGED_K, d["xg"]["q_colT"], d["xg"]["s_colT"], d["dym"]["q_colT"],
                           d["dym"]["s_colT"], d["dwm"], ge)

    bufs = [t for v in o.values() for t in (v.values() if isinstance(v, dict) else [v])]

    def zero_all():
        for t in bufs:
            t.zero_()

    zero_all()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in bufs]
    assert any(bool(t.any()) for t in ref)

    zero_all()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    # eager library work between replays, on buffers the graph does not use
    other = scaled_randn((M, K), 11).cuda()
    spare = _dual_bufs(m, M, K)
    for rep in range(3):
        zero_all()
        m.mxq_quantize(other, 3, spare["q_row"], spare["s_row"], spare["q_colT"], spare["s_colT"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(bufs, ref)):
            assert torch.equal(got, want), f"replay {rep}: buffer {i} {tuple(got.shape)} differs from the eager step"
    # and the eager step still gives the same after the replays
    zero_all()
    step()
    torch.cuda.synchronize()
    assert all(torch.equal(got, want) for got, want in zip(bufs, ref))
