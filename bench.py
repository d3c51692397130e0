"""Benchmark of the MX quantise + block-scaled GEMM hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * MXFP4 quant-dequant of an 8192x8192 fp32 tensor (1% of rows scaled by 2^U(-20,20));
  * MXFP8 dense linear M=8192, K=7168, N=18432: dual-axis quantisation of X and
    W, the forward GEMM, dual-axis quantisation of dY, then the input-gradient
    and weight-gradient GEMMs;
  * MoE expert layer, one GPU's 32 experts, 7168 -> 4096, 16384 tokens routed
    top-8 over Zipf(1.1) weights (131072 rows), dual-axis schedule: forward (X
    by rows, W[g] on both axes with the N-axis copy saved, ragged-M GEMM) and
    backward (dY by rows and grouped by tokens, X grouped by tokens, ragged-M
    input gradient, ragged-K weight gradient).
Timed beside the step, with the device memory each holds from forward to
backward: the MoE layer's forward/backward-split schedule (W[g] on its
reduction axis only in the forward, along N re-quantised in the backward)
and a dual schedule that also keeps X's token-axis copy from the forward; the
dense linear's two schedules; the MoE layer on the Zipf-law routing; the
MXFP4 QDQ with its saturation mask and the masked (clipped-STE) backward;
and the MXFP4 GEMMs (operand quantisation, the dense forward shape, the
ragged-M MoE forward shape and the ragged-K MoE weight gradient) with E2M1
operands.

Prints one JSON line.  `value` = GEMM FLOPs of the step / step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 GEMM & grouped-GEMM TFLOP/s (+quantize GB/s), % of MI355X roofline"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense FP4 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle CPU leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle leg")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for HBM counter scaling)")
    ap.add_argument("--quant-traffic", action="store_true",
                    help="only run each quantiser launch of the step once, in a fixed order, and print their "
                         "algorithmic bytes (for per-launch HBM counters)")
    return ap.parse_args()


PROFILE_DIR = os.path.join(ROOT, "profiles")
GEMM_SRC = os.path.join(ROOT, "moe_grouped_gemm_mxq_amd", "csrc", "gemm_mxfp8.hip")


def source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_label):
    """HBM bytes per launch of `kernel_label` from the committed counter summary,
    or None when there is none or the GEMM source changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"{kernel_label}__hbm_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel source sha256[:16]") != source_digest(GEMM_SRC):
        return None
    try:
        return int(float(vals["HBM bytes per launch"]))
    except (KeyError, ValueError):
        return None


class Timeline:
    """HIP events around each component on the launch stream."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def __call__(self, name):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(self.torch.cuda.current_stream())
        self.marks.append((name, ev))

    def durations(self):
        out = {}
        for (name, a), (_, b) in zip(self.marks, self.marks[1:]):
            if name is not None:
                out.setdefault(name, []).append(a.elapsed_time(b))
        return out


def moe_tile_stats(sizes, H, F, cus, BM=256, BN=256, BK=128):
    """Work the grouped GEMMs' tile walks do beyond the routed rows and tokens,
    and how evenly the persistent walks spread it over the workgroups (host
    arithmetic following the kernels' tiling: ragged-M tiles start at the
    128-row boundary at or below their group's first row; ragged-K tiles of a
    group reduce over its 32-padded tokens in 128-deep stages, an even number
    of them, from the 128-token boundary at or below the group's first padded
    position, and are dealt round robin, largest group first)."""
    out = {}
    # ragged M (forward: N = F; input gradient: N = H), K = H or F
    start, m_tiles = 0, 0
    for m in sizes:
        if m:
            m_tiles += (start - (start & ~127) + m + BM - 1) // BM
        start += m
    routed = sum(sizes)
    for name, n, k in (("raggedM_fwd", F, H), ("raggedM_dgrad", H, F)):
        tiles = m_tiles * ((n + BN - 1) // BN)
        rounds = -(-tiles // cus)
        out[name] = {"tiles": tiles, "rows_computed": m_tiles * BM, "rows_routed": routed,
                     "row_waste_frac": round(1 - routed / (m_tiles * BM), 4),
                     "max_over_mean_tiles_per_workgroup": round(rounds / (tiles / cus), 4)}
    # ragged K (weight gradient: M = H, N = F): the plain launch walks the
    # experts above 1024 tokens (their tiles' stages are 128 tokens deep, an
    # even number of them), the exact-group launch the others (empty ones
    # store zeros; a stage of 128 padded tokens runs one interleaved step per
    # 8 of them)
    per_g = ((H + BM - 1) // BM) * ((F + BN - 1) // BN)
    long_g = [g for g in range(len(sizes)) if sizes[g] > 1024]
    pos = [sum((m + 31) // 32 * 32 for m in sizes[:g]) for g in range(len(sizes))]  # padded group starts
    nst = {g: (-(-(pos[g] % BK + (sizes[g] + 31) // 32 * 32) // BK) + 1) // 2 * 2 for g in long_g}
    order = sorted(long_g, key=lambda g: (-sizes[g], g))
    work = [0] * cus
    tile = 0
    for g in order:
        for _ in range(per_g):
            work[tile % cus] += nst[g] + 1  # its stages plus one for the output tile
            tile += 1
    k_computed = sum(nst[g] * BK for g in long_g)
    routed_long = sum(sizes[g] for g in long_g)
    short = [g for g in range(len(sizes)) if sizes[g] <= 1024]
    out["raggedK_wgrad"] = {
        "plain_launch": {"experts": len(long_g), "tiles": tile, "tokens_routed": routed_long,
                         "tokens_computed": k_computed,
                         "token_waste_frac": round(1 - routed_long / k_computed, 4) if k_computed else 0.0,
                         "max_over_mean_stages_per_workgroup": round(max(work) / (sum(work) / cus), 4)
                         if tile else 0.0},
        "exact_group_launch": {"experts": len(short), "empty_experts": sum(1 for g in short if sizes[g] == 0),
                               "tiles": len(short) * per_g, "tokens_routed": sum(sizes[g] for g in short),
                               "interleaved_steps_per_tile": sum((sizes[g] + 31) // 32 * 4 for g in short)}}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the MX quantise/GEMM hot path on exactly one MI355X; runs on "
              "several GPUs are not part of this benchmark. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_grouped_gemm_mxq_amd import mxq, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": src.numel() * 4,
                          "bytes_written_per_launch": dst.numel() * 4, "launches": 5}))
        return
    if mxq.mxq_device_check(0) != mxq.MXQ_OK:
        raise RuntimeError(f"device 0 is not usable: {mxq.mxq_last_error()}")
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    c32 = lambda v: (v + 31) // 32 * 32

    # ---------------------------------------------------------------- inputs (resident)
    x4 = workloads.qdq_large().to(dev)
    y4 = torch.empty_like(x4)
    M, K, N = 8192, 7168, 18432
    X, W, dY = workloads.dense_linear(M, K, N, device=dev)
    Xm, Wm, dYm, ge = workloads.moe_layer(device=dev)
    ge = ge.to(dev)
    G, H, F = Wm.shape          # 32 experts, hidden 7168, ffn 4096
    T = Xm.shape[0]
    sizes = workloads.moe_group_sizes()

    # ---------------------------------------------------------------- outputs (allocated once)
    sc = lambda rows, nblk: u8(*mxq.scale_shape(rows, nblk))   # GEMM-operand scale array
    qx = dict(q_row=u8(M, K), s_row=sc(M, K // 32), q_colT=u8(K, M), s_colT=sc(K, M // 32))
    qw = dict(q_row=u8(K, N), s_row=sc(K, N // 32), q_colT=u8(N, K), s_colT=sc(N, K // 32))
    qy = dict(q_row=u8(M, N), s_row=sc(M, N // 32), q_colT=u8(N, M), s_colT=sc(N, M // 32))
    Y, dX, dW = f32(M, N), f32(M, K), f32(K, N)
    ldq = mxq.mxq_grouped_cols_max(T, G)
    mx = dict(q_row=u8(T, H), s_row=sc(T, H // 32))
    mw = dict(q_row=u8(G * H, F), s_row=sc(G * H, F // 32), q_colT=u8(G, F, H),
              s_colT=u8(G, *mxq.scale_shape(F, H // 32)))
    mdy = dict(q_row=u8(T, F), s_row=sc(T, F // 32), q_colT=u8(F, ldq), s_colT=sc(F, ldq // 32))
    mxt = dict(q_colT=u8(H, ldq), s_colT=sc(H, ldq // 32))
    mY, mdX, mdW = f32(T, F), f32(T, H), f32(G, H, F)
    R, C = mxq.MXQ_AXIS_ROW, mxq.MXQ_AXIS_COLT

    def quant_w_experts(mask):
        # all experts in one launch; the row copy / scales of expert g are rows
        # [g*H, (g+1)*H) of the stacked buffers (H is a multiple of 32)
        mxq.mxq_quantize_batched(Wm, mask,
                                 mw["q_row"].view(G, H, F) if mask & R else None,
                                 mw["s_row"].view(G, H // 128, F // 32, 32, 4) if mask & R else None,
                                 mw["q_colT"] if mask & C else None, mw["s_colT"] if mask & C else None)

    # Expert weights (MindSpeed PR 3852): the dual-axis schedule quantises
    # W[g] along K and along N from one read in the forward and keeps the
    # N-axis copy for the input gradient; fb-split quantises W[g] along K only
    # and re-quantises it along N in the backward.  In both, X is quantised by
    # rows in the forward and by tokens within each expert group in the
    # backward.  "dual_x" is the dual schedule that also quantises X by
    # tokens in the forward (one read of X for both copies) and keeps that
    # copy, as the dense dual schedule keeps X's column copy.
    def moe_fwd(tl, schedule, Xs=None, ges=None):
        Xs = Xm if Xs is None else Xs
        ges = ge if ges is None else ges
        if schedule == "dual_x":
            tl("moe_quant_x_row_grouped")
            mxq.mxq_quantize_grouped(Xs, ges, ldq, R | C, mx["q_row"], mx["s_row"], mxt["q_colT"], mxt["s_colT"])
        else:
            tl("moe_quant_x_row")
            mxq.mxq_quantize(Xs, R, mx["q_row"], mx["s_row"])
        tl("moe_quant_w_colT" if schedule == "fb_split" else "moe_quant_w_dual")
        quant_w_experts(C if schedule == "fb_split" else R | C)
        tl("moe_gemm_fwd_raggedM")
        mxq.mxq_grouped_gemm(mxq.MXQ_GG_RAGGED_M, mx["q_row"], mx["s_row"], mw["q_colT"], mw["s_colT"], mY, ges)

    def moe_bwd(tl, schedule, Xs=None, ges=None):
        Xs = Xm if Xs is None else Xs
        ges = ge if ges is None else ges
        tl("moe_quant_dy_row_grouped")
        mxq.mxq_quantize_grouped(dYm, ges, ldq, R | C, mdy["q_row"], mdy["s_row"], mdy["q_colT"], mdy["s_colT"])
        if schedule != "dual_x":
            tl("moe_quant_x_grouped")
            mxq.mxq_quantize_grouped(Xs, ges, ldq, C, None, None, mxt["q_colT"], mxt["s_colT"])
        if schedule == "fb_split":
            tl("moe_requant_w_row")
            quant_w_experts(R)
        tl("moe_gemm_dgrad_raggedM")
        mxq.mxq_grouped_gemm(mxq.MXQ_GG_RAGGED_M, mdy["q_row"], mdy["s_row"], mw["q_row"].view(G, H, F),
                             mw["s_row"].view(G, H // 128, F // 32, 32, 4), mdX, ges)
        tl("moe_gemm_wgrad_raggedK")
        mxq.mxq_grouped_gemm(mxq.MXQ_GG_RAGGED_K, mxt["q_colT"], mxt["s_colT"], mdy["q_colT"], mdy["s_colT"], mdW, ges)

    def step(tl):
        tl("qdq_fp4")
        mxq.mxq_qdq_fp4(x4, y4)
        # forward operands, forward GEMM, then the gradient's operands and the
        # backward GEMMs, in the order of a training step
        tl("dense_quant_dual_x_w")
        mxq.mxq_quantize(X, R | C, qx["q_row"], qx["s_row"], qx["q_colT"], qx["s_colT"])
        mxq.mxq_quantize(W, R | C, qw["q_row"], qw["s_row"], qw["q_colT"], qw["s_colT"])
        tl("dense_gemm_fwd")
        mxq.mxq_gemm(qx["q_row"], qx["s_row"], qw["q_colT"], qw["s_colT"], Y)
        tl("dense_quant_dual_dy")
        mxq.mxq_quantize(dY, R | C, qy["q_row"], qy["s_row"], qy["q_colT"], qy["s_colT"])
        tl("dense_gemm_dgrad")
        mxq.mxq_gemm(qy["q_row"], qy["s_row"], qw["q_row"], qw["s_row"], dX)
        tl("dense_gemm_wgrad")
        mxq.mxq_gemm(qx["q_colT"], qx["s_colT"], qy["q_colT"], qy["s_colT"], dW)
        moe_fwd(tl, "dual")
        moe_bwd(tl, "dual")
        tl(None)

    # ---------------------------------------------------------------- algorithmic work
    routed = sum(sizes)
    flops = {
        "dense_gemm_fwd": 2.0 * M * N * K, "dense_gemm_dgrad": 2.0 * M * N * K, "dense_gemm_wgrad": 2.0 * M * N * K,
        "moe_gemm_fwd_raggedM": 2.0 * routed * H * F, "moe_gemm_dgrad_raggedM": 2.0 * routed * H * F,
        "moe_gemm_wgrad_raggedK": 2.0 * routed * H * F,
    }
    qb = lambda r, c, n_axes: r * c * (2 + n_axes * (1 + 1 / 32))     # bf16 read once, codes+scales per axis
    padded = sum(c32(s) for s in sizes)
    bytes_ = {
        "qdq_fp4": 8.0 * x4.numel(),
        "dense_quant_dual_x_w": qb(M, K, 2) + qb(K, N, 2), "dense_quant_dual_dy": qb(M, N, 2),
        "moe_quant_x_row": qb(T, H, 1),
        "moe_quant_x_row_grouped": T * H * 2 + T * H * (1 + 1 / 32) + padded * H * (1 + 1 / 32),
        "moe_quant_w_dual": qb(G * H, F, 2),
        "moe_quant_w_colT": qb(G * H, F, 1),
        "moe_requant_w_row": qb(G * H, F, 1),
        "moe_quant_dy_row_grouped": T * F * 2 + T * F * (1 + 1 / 32) + padded * F * (1 + 1 / 32),
        "moe_quant_x_grouped": T * H * 2 + padded * H * (1 + 1 / 32),
    }
    step_flops = sum(flops.values())

    if args.quant_traffic:
        # every quantiser launch of the step once; the printed order is the
        # dispatch order of the quantiser kernels
        launches = []
        mxq.mxq_qdq_fp4(x4, y4)
        launches.append(["qdq_fp4 8192x8192", "qdq_flat_kernel", bytes_["qdq_fp4"]])
        for name, t, q, r, c in (("X", X, qx, M, K), ("W", W, qw, K, N), ("dY", dY, qy, M, N)):
            mxq.mxq_quantize(t, R | C, q["q_row"], q["s_row"], q["q_colT"], q["s_colT"])
            launches.append([f"dense_quant_dual {name} {r}x{c}", "quant_tile_kernel<true, true>", qb(r, c, 2)])
        mxq.mxq_quantize(Xm, R, mx["q_row"], mx["s_row"])
        launches.append([f"moe_quant_x_row {T}x{H}", "quant_row_kernel<true>", bytes_["moe_quant_x_row"]])
        quant_w_experts(R | C)
        launches.append([f"moe_quant_w_dual {G}x{H}x{F}", "quant_tile_kernel<true, true>",
                         bytes_["moe_quant_w_dual"]])
        mxq.mxq_quantize_grouped(dYm, ge, ldq, R | C, mdy["q_row"], mdy["s_row"], mdy["q_colT"], mdy["s_colT"])
        launches.append([f"moe_quant_dy_row_grouped {T}x{F}", "quant_tile_grouped_kernel<true, true>",
                         bytes_["moe_quant_dy_row_grouped"]])
        mxq.mxq_quantize_grouped(Xm, ge, ldq, C, None, None, mxt["q_colT"], mxt["s_colT"])
        launches.append([f"moe_quant_x_grouped {T}x{H}", "quant_tile_grouped_kernel<false, true>",
                         bytes_["moe_quant_x_grouped"]])
        # beside the step: the dual_x schedule's X launch (rows and tokens from one read)
        mxq.mxq_quantize_grouped(Xm, ge, ldq, R | C, mx["q_row"], mx["s_row"], mxt["q_colT"], mxt["s_colT"])
        launches.append([f"moe_quant_x_row_grouped {T}x{H} (dual_x forward)", "quant_tile_grouped_kernel<true, true>",
                         bytes_["moe_quant_x_row_grouped"]])
        # beside the step: the MXFP4 operand quantisers of the MXFP4 GEMMs (fp32
        # inputs): the dense forward's X and W^T by rows, the MoE weight
        # gradient's X and dY along each expert's tokens
        for name, t in (("X", X.float()), ("W^T", W.t().contiguous().float())):
            mxq.quantize_fp4(t)
            r, c = t.shape
            launches.append([f"mxfp4_operand {name} {r}x{c}", "quant_fp4_rows_kernel", r * c * (4 + 0.5 + 1 / 32)])
            del t
        for name, t in (("X", Xm.float()), ("dY", dYm.float())):
            mxq.quantize_fp4_grouped(t, ge, ldq)
            c = t.shape[1]
            launches.append([f"mxfp4_token_axis {name} {T}x{c}", "quant_fp4_grouped_kernel<true>",
                             T * c * 4 + padded * c * (0.5 + 1 / 32)])
            del t
        torch.cuda.synchronize()
        print(json.dumps({"quant_traffic_launches": launches}))
        return

    # ---------------------------------------------------------------- warmup + timed steps
    for _ in range(args.warmup):
        step(Timeline(torch))
    torch.cuda.synchronize()
    tls = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        tl = Timeline(torch)
        step(tl)
        tls.append(tl)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    per = {}
    for tl in tls:
        for k, v in tl.durations().items():
            per.setdefault(k, []).extend(v)
    avg = {k: sum(v) / len(v) for k, v in per.items()}
    components = {}
    for k, ms in avg.items():
        d = {"ms": round(ms, 4)}
        if k in flops:
            tf = flops[k] / (ms * 1e-3) / 1e12
            d.update(tflops=round(tf, 1), frac_fp8_peak=round(tf / PEAK_FP8_TFLOPS, 4))
        if k in bytes_:
            gbs = bytes_[k] / (ms * 1e-3) / 1e9
            d.update(gbs=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))
        components[k] = d

    # GEMM kernels of the step and the components (one launch each) they run
    kernels = {
        "moe_gemm_raggedM": ("gemm_mx_kernel ragged M (expert forward and input gradient)",
                             ["moe_gemm_fwd_raggedM", "moe_gemm_dgrad_raggedM"]),
        "dense_gemm": ("gemm_mx_kernel dense (forward, input and weight gradient)",
                       ["dense_gemm_fwd", "dense_gemm_dgrad", "dense_gemm_wgrad"]),
        "moe_gemm_wgrad_raggedK": ("gemm_mx_kernel ragged K (expert weight gradient; experts with more than "
                                   "1024 tokens, then the exact-group launch for the rest)",
                                   ["moe_gemm_wgrad_raggedK"]),
    }

    def kernel_roofline(label):
        desc, comps = kernels[label]
        launch_ms = sum(avg[c] for c in comps) / len(comps)        # mean over its launches
        per_launch = sum(flops[c] for c in comps) / len(comps)     # (equal FLOPs per launch)
        tf = per_launch / (launch_ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": label, "description": desc, "achieved": round(tf, 1),
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                "traffic": measured_traffic(label), "algorithmic_flops_per_launch": per_launch,
                "avg_launch_ms": round(launch_ms, 4), "launches_per_step": len(comps),
                "step_share": round(sum(avg[c] for c in comps) / ms_per_step, 4)}

    # dominant kernel: the GEMM kernel with the largest share of the step;
    # beside it the slowest single launch
    dom = max(kernels, key=lambda k: sum(avg[c] for c in kernels[k][1]))
    slow = max(kernels, key=lambda k: max(avg[c] for c in kernels[k][1]))
    roofline = kernel_roofline(dom)
    roofline_slowest = kernel_roofline(slow)

    # ---------------------------------------------------------------- dense schedules: time and memory
    # dual: the forward quantises X and W on both axes and keeps X's column
    # copy and W's row copy for the backward; fb-split: the forward quantises
    # only what it uses (X rows, W columns) and the backward re-quantises X
    # along M and W along N from bf16 (MindSpeed PR 3852, fp8-quant-fb-split).
    def dense_fwd(sched):
        if sched == "dual":
            mxq.mxq_quantize(X, R | C, qx["q_row"], qx["s_row"], qx["q_colT"], qx["s_colT"])
            mxq.mxq_quantize(W, R | C, qw["q_row"], qw["s_row"], qw["q_colT"], qw["s_colT"])
        else:
            mxq.mxq_quantize(X, R, qx["q_row"], qx["s_row"])
            mxq.mxq_quantize(W, C, None, None, qw["q_colT"], qw["s_colT"])
        mxq.mxq_gemm(qx["q_row"], qx["s_row"], qw["q_colT"], qw["s_colT"], Y)

    def dense_bwd(sched):
        if sched == "fb_split":
            mxq.mxq_quantize(X, C, None, None, qx["q_colT"], qx["s_colT"])
            mxq.mxq_quantize(W, R, qw["q_row"], qw["s_row"])
        mxq.mxq_quantize(dY, R | C, qy["q_row"], qy["s_row"], qy["q_colT"], qy["s_colT"])
        mxq.mxq_gemm(qy["q_row"], qy["s_row"], qw["q_row"], qw["s_row"], dX)
        mxq.mxq_gemm(qx["q_colT"], qx["s_colT"], qy["q_colT"], qy["s_colT"], dW)

    def time_schedule(fwd, bwd, sched):
        for _ in range(2):
            fwd(sched)
            bwd(sched)
        torch.cuda.synchronize()
        fb = []
        for _ in range(5):
            tl = Timeline(torch)
            tl("fwd")
            fwd(sched)
            tl("bwd")
            bwd(sched)
            tl(None)
            fb.append(tl)
        torch.cuda.synchronize()
        d = {}
        for tl in fb:
            for k, v in tl.durations().items():
                d.setdefault(k, []).extend(v)
        return round(sum(d["fwd"]) / len(d["fwd"]), 3), round(sum(d["bwd"]) / len(d["bwd"]), 3)

    dense_sched = {}
    grads = {}
    for sched in ("dual", "fb_split"):
        f_ms, b_ms = time_schedule(dense_fwd, dense_bwd, sched)
        held = (qx["q_colT"].numel() + qx["s_colT"].numel() + qw["q_row"].numel() + qw["s_row"].numel()
                if sched == "dual" else 0)
        dense_sched[sched] = {"fwd_ms": f_ms, "bwd_ms": b_ms, "quantised_held_fwd_to_bwd_bytes": held}
        grads[sched] = (dX.clone(), dW.clone())
    # measured device memory of each schedule (untimed; as for the MoE layer
    # below): every quantised copy allocated when produced, freed after its
    # last use
    def dense_memory(sched):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        both = R | C if sched == "dual" else None
        xq = mxq.quantize(X, both or R)
        wq = mxq.quantize(W, both or C)
        mxq.mxq_gemm(xq["q_row"], xq["s_row"], wq["q_colT"], wq["s_colT"], Y)
        for k in ("q_row", "s_row"):
            del xq[k]
        for k in ("q_colT", "s_colT"):
            del wq[k]
        torch.cuda.synchronize()
        held = torch.cuda.memory_allocated() - base
        if sched == "fb_split":
            xq.update(mxq.quantize(X, C))
            wq.update(mxq.quantize(W, R))
        yq = mxq.quantize(dY, R | C)
        mxq.mxq_gemm(yq["q_row"], yq["s_row"], wq["q_row"], wq["s_row"], dX)
        mxq.mxq_gemm(xq["q_colT"], xq["s_colT"], yq["q_colT"], yq["s_colT"], dW)
        del xq, wq, yq
        torch.cuda.synchronize()
        return {"held_fwd_to_bwd_bytes": held, "fwd_bwd_peak_bytes": torch.cuda.max_memory_allocated() - base}

    for sched in ("dual", "fb_split"):
        dense_sched[sched]["measured_memory"] = dense_memory(sched)
    dense_sched["bitwise_equal_grads"] = bool(torch.equal(grads["dual"][0], grads["fb_split"][0]) and
                                              torch.equal(grads["dual"][1], grads["fb_split"][1]))
    del grads

    # ---------------------------------------------------------------- clipped-STE fake quantiser
    # MXFP4 QDQ that also writes the saturation bitmask (one bit per element),
    # then the masked backward, on the same 8192x8192 tensor; y4 stands in for
    # the incoming gradient.
    mask4 = u8(x4.shape[0], x4.shape[1] // 8)
    gx4 = torch.empty_like(x4)
    n4 = x4.numel()
    ste_bytes = {"fwd_qdq_with_mask": 8.0 * n4 + n4 / 8, "bwd_masked_grad": 8.0 * n4 + n4 / 8}
    ste_runs = []
    for i in range(12):
        tl = Timeline(torch)
        tl("fwd_qdq_with_mask")
        mxq.mxq_qdq_fp4_ex(x4, y4, 6.0, None, None, mask4)
        tl("bwd_masked_grad")
        mxq.mxq_ste_backward_fp4(y4, mask4, gx4)
        tl(None)
        if i >= 2:
            ste_runs.append(tl)
    torch.cuda.synchronize()
    fake_quant = {}
    for tl in ste_runs:
        for k, v in tl.durations().items():
            fake_quant.setdefault(k, []).extend(v)
    for k, v in list(fake_quant.items()):
        ms = sum(v) / len(v)
        gbs = ste_bytes[k] / (ms * 1e-3) / 1e9
        fake_quant[k] = {"ms": round(ms, 4), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}

    # ---------------------------------------------------------------- MXFP4 GEMM
    # The dense linear's forward shape with E2M1 operands: X [M][K] and W^T
    # [N][K] in fp32, quantised to MXFP4 GEMM operands, then the FP4 GEMM.
    xf = X.float()
    wtf = W.t().contiguous().float()
    qa, sa = mxq.quantize_fp4(xf)
    qb, sb = mxq.quantize_fp4(wtf)
    Y4 = f32(M, N)
    fp4_runs = []
    for i in range(8):
        tl = Timeline(torch)
        tl("quant_fp4_operands")
        mxq.mxq_quantize_fp4(xf, qa, sa)
        mxq.mxq_quantize_fp4(wtf, qb, sb)
        tl("gemm_fp4")
        mxq.mxq_gemm(qa, sa, qb, sb, Y4, fmt=mxq.MXQ_FMT_E2M1)
        tl(None)
        if i >= 2:
            fp4_runs.append(tl)
    torch.cuda.synchronize()
    d4 = {}
    for tl in fp4_runs:
        for k, v in tl.durations().items():
            d4.setdefault(k, []).extend(v)
    g_ms = sum(d4["gemm_fp4"]) / len(d4["gemm_fp4"])
    q_ms = sum(d4["quant_fp4_operands"]) / len(d4["quant_fp4_operands"])
    g_tf = 2.0 * M * N * K / (g_ms * 1e-3) / 1e12
    q_gbs = (M + N) * K * (4 + 0.5 + 1 / 32) / (q_ms * 1e-3) / 1e9
    mxfp4_gemm = {"shape": f"M{M} N{N} K{K}", "gemm_ms": round(g_ms, 4), "gemm_tflops": round(g_tf, 1),
                  "frac_fp4_peak": round(g_tf / PEAK_FP4_TFLOPS, 4), "quant_ms": round(q_ms, 4),
                  "quant_gbs": round(q_gbs, 1), "quant_frac_hbm_peak": round(q_gbs / PEAK_HBM_GBS, 4)}
    del xf, wtf, qa, sa, qb, sb, Y4

    # The MoE forward shape with E2M1 operands: the routed token rows and every
    # expert's W[g]^T [F][H] in fp32, quantised to MXFP4 GEMM operands, then
    # the ragged-M FP4 GEMM over the same expert groups.
    xmf = Xm.float()
    qxm, sxm = mxq.quantize_fp4(xmf)
    del xmf
    wmf = Wm.transpose(1, 2).reshape(G * F, H).float()
    qwm, swm = mxq.quantize_fp4(wmf)
    del wmf
    qwm = qwm.view(G, F, H // 2)
    swm = swm.view(G, F // 128, H // 32, 32, 4)
    moe4_runs = []
    for i in range(6):
        tl = Timeline(torch)
        tl("gemm_fp4_raggedM")
        mxq.mxq_grouped_gemm(mxq.MXQ_GG_RAGGED_M, qxm, sxm, qwm, swm, mY, ge, fmt=mxq.MXQ_FMT_E2M1)
        tl(None)
        if i >= 2:
            moe4_runs.append(tl)
    torch.cuda.synchronize()
    m4 = [v for tl in moe4_runs for v in tl.durations()["gemm_fp4_raggedM"]]
    m4_ms = sum(m4) / len(m4)
    m4_tf = 2.0 * routed * H * F / (m4_ms * 1e-3) / 1e12
    mxfp4_moe_gemm = {"shape": f"{routed} routed rows, {G} experts, {H} -> {F}", "gemm_ms": round(m4_ms, 4),
                      "gemm_tflops": round(m4_tf, 1), "frac_fp4_peak": round(m4_tf / PEAK_FP4_TFLOPS, 4)}
    del qxm, sxm, qwm, swm

    # The MoE weight gradient with E2M1 operands: the fp32 token rows and dY
    # quantised along the token axis within each expert group, then the
    # ragged-K FP4 GEMM into every expert's dW.
    xmf, dymf = Xm.float(), dYm.float()
    gx4 = mxq.quantize_fp4_grouped(xmf, ge, ldq)
    gy4 = mxq.quantize_fp4_grouped(dymf, ge, ldq)
    wg4_runs = []
    for i in range(6):
        tl = Timeline(torch)
        tl("quant_fp4_token_axis")
        mxq.mxq_quantize_fp4_grouped(xmf, ge, ldq, gx4["codes"], gx4["scales"])
        mxq.mxq_quantize_fp4_grouped(dymf, ge, ldq, gy4["codes"], gy4["scales"])
        tl("gemm_fp4_raggedK")
        mxq.mxq_grouped_gemm(mxq.MXQ_GG_RAGGED_K, gx4["codes"], gx4["scales"], gy4["codes"], gy4["scales"], mdW, ge,
                             fmt=mxq.MXQ_FMT_E2M1)
        tl(None)
        if i >= 2:
            wg4_runs.append(tl)
    torch.cuda.synchronize()
    dw4 = {}
    for tl in wg4_runs:
        for k, v in tl.durations().items():
            dw4.setdefault(k, []).extend(v)
    w4_ms = sum(dw4["gemm_fp4_raggedK"]) / len(dw4["gemm_fp4_raggedK"])
    q4_ms = sum(dw4["quant_fp4_token_axis"]) / len(dw4["quant_fp4_token_axis"])
    w4_tf = 2.0 * routed * H * F / (w4_ms * 1e-3) / 1e12
    q4_bytes = T * (H + F) * 4 + padded * (H + F) * (0.5 + 1 / 32)
    mxfp4_moe_wgrad = {"shape": f"{routed} routed rows, {G} experts, dW {H} x {F} each",
                       "gemm_ms": round(w4_ms, 4), "gemm_tflops": round(w4_tf, 1),
                       "frac_fp4_peak": round(w4_tf / PEAK_FP4_TFLOPS, 4), "quant_ms": round(q4_ms, 4),
                       "quant_gbs": round(q4_bytes / (q4_ms * 1e-3) / 1e9, 1),
                       "quant_frac_hbm_peak": round(q4_bytes / (q4_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del xmf, dymf, gx4, gy4

    # ---------------------------------------------------------------- MoE schedules: time and memory
    schedules = {}
    for sched in ("dual", "fb_split", "dual_x"):
        for _ in range(2):
            tl = Timeline(torch)
            moe_fwd(tl, sched)
            moe_bwd(tl, sched)
            tl(None)
        torch.cuda.synchronize()
        fb = []
        for _ in range(5):
            tl = Timeline(torch)
            tl("fwd")
            moe_fwd(Timeline(torch), sched)
            tl("bwd")
            moe_bwd(Timeline(torch), sched)
            tl(None)
            fb.append(tl)
        torch.cuda.synchronize()
        d = {}
        for tl in fb:
            for k, v in tl.durations().items():
                d.setdefault(k, []).extend(v)
        held_w = (mw["q_row"].numel() + mw["s_row"].numel()) if sched != "fb_split" else 0
        held_x = (mxt["q_colT"].numel() + mxt["s_colT"].numel()) if sched == "dual_x" else 0
        schedules[sched] = {"fwd_ms": round(sum(d["fwd"]) / len(d["fwd"]), 3),
                            "bwd_ms": round(sum(d["bwd"]) / len(d["bwd"]), 3),
                            "quantised_w_held_fwd_to_bwd_bytes": held_w,
                            "quantised_x_held_fwd_to_bwd_bytes": held_x}
    # Measured device memory of each schedule (untimed): one MoE forward and
    # backward in which every quantised copy is allocated when it is produced
    # and freed after its last use, as a training step would.  `held` = bytes
    # still allocated when the forward ends (the saved W row copy of the dual
    # schedule), `peak` = the peak over forward and backward, both relative to
    # the allocations before the forward (caching-allocator counters).
    def moe_memory(sched):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        xq = mxq.quantize_grouped(Xm, ge, R | C, ldq) if sched == "dual_x" else mxq.quantize(Xm, R)
        wq = mxq.quantize_batched(Wm, C if sched == "fb_split" else R | C)
        mxq.mxq_grouped_gemm(mxq.MXQ_GG_RAGGED_M, xq["q_row"], xq["s_row"], wq["q_colT"], wq["s_colT"], mY, ge)
        for k in ("q_row", "s_row"):
            del xq[k]
        del wq["q_colT"], wq["s_colT"]
        torch.cuda.synchronize()
        held = torch.cuda.memory_allocated() - base
        fwd_peak = torch.cuda.max_memory_allocated() - base
        dyq = mxq.quantize_grouped(dYm, ge, R | C, ldq)
        xt = xq if sched == "dual_x" else mxq.quantize_grouped(Xm, ge, C, ldq)
        if sched == "fb_split":
            wq.update(mxq.quantize_batched(Wm, R))
        mxq.mxq_grouped_gemm(mxq.MXQ_GG_RAGGED_M, dyq["q_row"], dyq["s_row"], wq["q_row"], wq["s_row"], mdX, ge)
        mxq.mxq_grouped_gemm(mxq.MXQ_GG_RAGGED_K, xt["q_colT"], xt["s_colT"], dyq["q_colT"], dyq["s_colT"], mdW, ge)
        del dyq, xt, xq, wq
        torch.cuda.synchronize()
        return {"held_fwd_to_bwd_bytes": held, "fwd_peak_bytes": fwd_peak,
                "fwd_bwd_peak_bytes": torch.cuda.max_memory_allocated() - base}

    for sched in ("dual", "fb_split", "dual_x"):
        schedules[sched]["measured_memory"] = moe_memory(sched)
    schedules["measured_held_difference_bytes"] = (schedules["dual"]["measured_memory"]["held_fwd_to_bwd_bytes"] -
                                                   schedules["fb_split"]["measured_memory"]["held_fwd_to_bwd_bytes"])

    # the schedules must produce the same input and weight gradients bit for bit
    grads = {}
    for sched in ("dual", "fb_split", "dual_x"):
        moe_fwd(Timeline(torch), sched)
        moe_bwd(Timeline(torch), sched)
        grads[sched] = (mdX.clone(), mdW.clone())
    torch.cuda.synchronize()
    schedules["bitwise_equal_dgrad"] = all(torch.equal(grads["dual"][0], g[0]) for g in grads.values())
    schedules["bitwise_equal_wgrad"] = all(torch.equal(grads["dual"][1], g[1]) for g in grads.values())
    del grads

    # ---------------------------------------------------------------- Zipf-law routing
    # The same layer with tokens routed over Zipf-law expert popularity
    # (e + 1)^-1.1: no empty expert, every size off a multiple of 32.  X and
    # dY are the same draws as above, X gathered in this routing's expert
    # order; the dual schedule, per-component times.
    Xl, _, _, gel = workloads.moe_layer(device=dev, with_dy=False, routing="zipf_law")
    gel = gel.to(dev)
    law_runs = []
    for i in range(6):
        tl = Timeline(torch)
        moe_fwd(tl, "dual", Xl, gel)
        moe_bwd(tl, "dual", Xl, gel)
        tl(None)
        if i >= 2:
            law_runs.append(tl)
    torch.cuda.synchronize()
    dl = {}
    for tl in law_runs:
        for k, v in tl.durations().items():
            dl.setdefault(k, []).extend(v)
    law_sizes = workloads.moe_group_sizes("zipf_law")
    law = {"sizes": law_sizes, "components": {}}
    for k, v in dl.items():
        ms = sum(v) / len(v)
        d = {"ms": round(ms, 4)}
        if k.startswith("moe_gemm"):
            tf = 2.0 * T * H * F / (ms * 1e-3) / 1e12
            d.update(tflops=round(tf, 1), frac_fp8_peak=round(tf / PEAK_FP8_TFLOPS, 4))
        law["components"][k] = d
    law["fwd_bwd_ms"] = round(sum(d["ms"] for d in law["components"].values()), 3)
    law["tiles"] = moe_tile_stats(law_sizes, H, F, torch.cuda.get_device_properties(0).multi_processor_count)
    del Xl, gel

    # ---------------------------------------------------------------- small linear forward
    # X [256x512] and W [512x256] (N(0,1), seed 0): quantise X by rows and W
    # by columns, then the GEMM into a [256x256] fp32 output.  Latency-bound
    # (67.1 MFLOP); 100 timed repetitions after 10, median of each part.
    Xs, Ws = workloads.linear_small(device=dev)
    qxs = mxq.quantize(Xs, R)
    qws = mxq.quantize(Ws, C)
    Ys = f32(Xs.shape[0], Ws.shape[1])
    small = {"quant_x_row": [], "quant_w_colT": [], "gemm": [], "total": []}
    for i in range(110):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        mxq.mxq_quantize(Xs, R, qxs["q_row"], qxs["s_row"])
        ev[1].record()
        mxq.mxq_quantize(Ws, C, None, None, qws["q_colT"], qws["s_colT"])
        ev[2].record()
        mxq.mxq_gemm(qxs["q_row"], qxs["s_row"], qws["q_colT"], qws["s_colT"], Ys)
        ev[3].record()
        if i >= 10:
            small["_ev"] = small.get("_ev", []) + [ev]
    torch.cuda.synchronize()
    for ev in small.pop("_ev"):
        small["quant_x_row"].append(ev[0].elapsed_time(ev[1]))
        small["quant_w_colT"].append(ev[1].elapsed_time(ev[2]))
        small["gemm"].append(ev[2].elapsed_time(ev[3]))
        small["total"].append(ev[0].elapsed_time(ev[3]))
    med = lambda v: sorted(v)[len(v) // 2]
    linear_small = {"shape": "X 256x512 . W 512x256 -> 256x256 fp32", "reps": len(small["total"])}
    for k, v in small.items():
        linear_small[f"{k}_us_median"] = round(1e3 * med(v), 2)
    linear_small["gemm_tflops_median"] = round(2.0 * 256 * 256 * 512 / (med(small["gemm"]) * 1e-3) / 1e12, 2)
    del Xs, Ws, qxs, qws, Ys

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds, X, W, dY, Xm, Wm, dYm, ge, sizes, x4)

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) activations and gradients, N(0,0.02^2) weights, "
                "Zipf(1.1) top-8 routing; MXFP4 input N(0,1) with 1% rows x 2^U(-20,20))",
        "config": {
            "workload": "MX hot path step: MXFP4 QDQ 8192x8192 fp32 + MXFP8 dense linear M8192 K7168 N18432 "
                        "fwd/dgrad/wgrad with dual-axis quantisation + MoE 32 experts x (7168->4096), "
                        "131072 routed rows, fwd/bwd, dual-axis schedule (W[g] quantised on both axes in the forward, "
                        "its N-axis copy saved; X by rows in the forward and by tokens in the backward)",
            "gemm_tflop_per_step": round(step_flops / 1e12, 3),
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "roofline_slowest_launch": roofline_slowest,
        "cpu_baseline": cpu,
        "components": components,
        "dense_schedules": dense_sched,
        "mxfp4_clipped_ste": fake_quant,
        "mxfp4_gemm": mxfp4_gemm,
        "mxfp4_moe_gemm": mxfp4_moe_gemm,
        "mxfp4_moe_wgrad": mxfp4_moe_wgrad,
        "moe_schedules": schedules,
        "moe_zipf_law_routing": law,
        "moe_tiles": moe_tile_stats(sizes, H, F, torch.cuda.get_device_properties(0).multi_processor_count),
        "linear_small": linear_small,
    }
    print(json.dumps(out))


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(target_s, X, W, dY, Xm, Wm, dYm, ge, sizes, x4):
    """The oracle (plain C, fp64) on a bounded sample of the same workload: for
    each of the six GEMMs, quantise the operand rows/columns a block of sampled
    outputs needs and compute those outputs; TFLOP/s = sampled GEMM FLOPs /
    oracle time (quantisation included)."""
    import numpy as np
    import torch
    import oracle
    from moe_grouped_gemm_mxq_amd.workloads import bf16_bits

    rows = lambda t, idx: bf16_bits(t[torch.as_tensor(idx, device=t.device)])
    cols = lambda t, idx: np.ascontiguousarray(bf16_bits(t[:, torch.as_tensor(idx, device=t.device)].contiguous()).T)
    ge_np = ge.cpu().numpy()
    big = int(np.argmax(sizes))
    start = int(ge_np[big - 1]) if big else 0
    rng = np.random.default_rng(0)

    def gather(s):
        """(A-source rows, B-source rows, K) of the sampled block for each GEMM, s x s outputs."""
        mi = rng.choice(X.shape[0], s, replace=False)
        ni = rng.choice(W.shape[1], s, replace=False)
        ki = rng.choice(W.shape[0], s, replace=False)
        ti = start + rng.choice(sizes[big], s, replace=False)
        fi = rng.choice(Wm.shape[2], s, replace=False)
        hi = rng.choice(Wm.shape[1], s, replace=False)
        return [
            (lambda: rows(X, mi), lambda: cols(W, ni)),            # dense fwd, K = 7168
            (lambda: rows(dY, mi), lambda: rows(W, ki)),            # dense dgrad, K = 18432
            (lambda: cols(X, ki), lambda: cols(dY, ni)),            # dense wgrad, K = 8192
            (lambda: rows(Xm, ti), lambda: cols(Wm[big], fi)),      # MoE fwd (largest expert), K = 7168
            (lambda: rows(dYm, ti), lambda: rows(Wm[big], hi)),     # MoE dgrad, K = 4096
            (lambda: cols(Xm[start:start + sizes[big]], hi),        # MoE wgrad of that expert, K = its tokens
             lambda: cols(dYm[start:start + sizes[big]], fi)),
        ]

    def run(s):
        work = gather(s)
        srcs = [(fa(), fb()) for fa, fb in work]     # host copies of the bf16 inputs (not timed)
        t0 = time.perf_counter()
        fl = 0.0
        for a_bits, b_bits in srcs:
            A, sA = oracle.mxfp8_quant_row(a_bits)
            B, sB = oracle.mxfp8_quant_row(b_bits)
            oracle.gemm(A, sA, B, sB)
            fl += 2.0 * A.shape[0] * B.shape[0] * A.shape[1]
        return time.perf_counter() - t0, fl

    def grow(target):
        # grow the sample (cost ~ s^2) until one run takes about `target` seconds
        s = 64
        t, fl = run(s)
        while t < 0.5 * target and s < 4096:
            s = int(min(4096, s * max(1.4, min(4.0, (target / max(t, 1e-3)) ** 0.5))))
            t, fl = run(s)
        return s, t, fl

    def qdq_rate(target):
        # the MXFP4 QDQ oracle over leading rows of the 8192 x 8192 input,
        # doubling them until a run takes about `target` seconds; GB/s over
        # the same 8 bytes per element as the kernel (fp32 in, fp32 out)
        n = 64
        while True:
            xs = x4[:n].cpu().numpy()
            t0 = time.perf_counter()
            oracle.mxfp4_qdq(xs)
            t = time.perf_counter() - t0
            if t >= 0.5 * target or n >= x4.shape[0]:
                return n, t, 8.0 * xs.size / t / 1e9
            n = min(x4.shape[0], n * 2)

    def linear_small_rate(target):
        # the small linear forward (X [256x512] rows, W [512x256] columns, the
        # 256x256x512 GEMM) end to end in the oracle, repeated for about
        # `target` seconds; ms per forward and TFLOP/s over its 67.1 MFLOP
        from moe_grouped_gemm_mxq_amd.workloads import linear_small
        xs, ws = linear_small()
        xb, wb = bf16_bits(xs), bf16_bits(ws)
        n, t0 = 0, time.perf_counter()
        while True:
            A, sA = oracle.mxfp8_quant_row(xb)
            B, sB = oracle.mxfp8_quant_colT(wb)
            oracle.gemm(A, sA, B, sB)
            n += 1
            t = time.perf_counter() - t0
            if t >= target:
                break
        ms = 1e3 * t / n
        return {"ms_per_forward": round(ms, 3), "tflops": round(2.0 * 256 * 256 * 512 / (ms * 1e-3) / 1e12, 6),
                "reps": n}

    def dual_rate():
        # the MXFP8 dual-axis quantisation oracle (row copy + column copy) of
        # the dense X [8192 x 7168] bf16, over the kernel's 4.0625 bytes per
        # element (2 read, 2 x (1 + 1/32) written)
        xb = bf16_bits(X)
        t0 = time.perf_counter()
        oracle.mxfp8_quant_row(xb)
        oracle.mxfp8_quant_colT(xb)
        t = time.perf_counter() - t0
        return t, 4.0625 * xb.size / t / 1e9

    lib = oracle.lib()
    cores = lib.oracle_num_threads()
    s, t, fl = grow(target_s)
    qn, qt, qgbs = qdq_rate(0.15 * target_s)
    dt, dgbs = dual_rate()
    c0 = linear_small_rate(0.05 * target_s)
    lib.oracle_set_num_threads(1)
    try:
        s1, t1, fl1 = grow(0.3 * target_s)
        qn1, qt1, qgbs1 = qdq_rate(0.1 * target_s)
        c01 = linear_small_rate(0.05 * target_s)
    finally:
        lib.oracle_set_num_threads(cores)
    return {"value": round(fl / t / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{s}x{s} outputs of each of the six GEMMs (dense fwd/dgrad/wgrad; MoE fwd/dgrad/wgrad of "
                      f"the largest expert), with the oracle quantising the operand rows they need; "
                      f"{fl / 1e9:.1f} GFLOP in {t:.1f} s",
            "single_thread": {"value": round(fl1 / t1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                              "sample": f"{s1}x{s1} outputs of each of the six GEMMs; {fl1 / 1e9:.1f} GFLOP in "
                                        f"{t1:.1f} s"},
            "mxfp4_qdq": {"value": round(qgbs, 3), "unit": "GB/s", "cores": cores,
                          "sample": f"first {qn} rows of the 8192x8192 input, 8 bytes per element, {qt:.2f} s",
                          "single_thread": {"value": round(qgbs1, 3), "unit": "GB/s", "cores": 1,
                                            "sample": f"first {qn1} rows, {qt1:.2f} s"}},
            "linear_small": {"workload": "X 256x512 rows, W 512x256 columns, GEMM 256x256x512 (whole forward)",
                             "all_cores": {**c0, "cores": cores}, "single_thread": {**c01, "cores": 1}},
            "mxfp8_quantize_dual": {"value": round(dgbs, 3), "unit": "GB/s", "cores": cores,
                                    "sample": f"dense X {X.shape[0]}x{X.shape[1]} bf16, row and column copies, "
                                              f"4.0625 bytes per element, {dt:.2f} s"}}


if __name__ == "__main__":
    main()
