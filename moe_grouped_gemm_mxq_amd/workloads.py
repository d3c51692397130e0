"""Seeded synthetic inputs for the MX quantise / block-scaled GEMM hot path.

This module only draws random numbers and arranges them; it holds none of
the method's arithmetic (no scaling, rounding or products), so the oracle
side and the HIP side can both take their inputs from it.

Workloads (shapes and distributions of the sources' configurations):

* ``linear_small``  -- MXFP8 linear forward: X bf16 [256x512], W bf16
  [512x256], both N(0,1), seed 0.
* ``qdq_small`` / ``qdq_large`` -- MXFP4 quant-dequant inputs: fp32 (2,33),
  (3,17), (4,48,33) N(0,1); and [8192x8192] N(0,1) with 1% of the rows
  multiplied by 2^u, u ~ U(-20, 20).
* ``dense_linear`` -- MXFP8 dense linear fwd/dgrad/wgrad: X [8192x7168]
  N(0,1), W [7168x18432] N(0, 0.02^2), dY [8192x18432] N(0,1), all bf16.
* ``moe_*`` -- MoE expert layer (one GPU's 32 local experts): 16384 tokens,
  each routed to 8 distinct experts drawn by multinomial sampling over
  Zipf(1.1) expert weights; X = tokens [16384x7168] N(0,1) gathered in expert
  order into [131072x7168]; W [32x7168x4096] N(0, 0.02^2); dY [131072x4096]
  N(0,1); all bf16.  The per-expert row counts are frozen in
  ``data/moe_group_sizes_zipf1.1_top8.json``.  A second routing,
  ``routing="zipf_law"``, draws from Zipf-law expert popularity
  w_e = (e + 1)^-1.1 instead (every expert gets tokens); its sizes are
  frozen in ``data/moe_group_sizes_zipflaw1.1_top8.json``.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

_DATA = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data")
MOE_SIZES_FILE = os.path.join(_DATA, "moe_group_sizes_zipf1.1_top8.json")
MOE_LAW_SIZES_FILE = os.path.join(_DATA, "moe_group_sizes_zipflaw1.1_top8.json")
ROUTINGS = ("zipf_weights", "zipf_law")

MOE_EXPERTS = 32
MOE_TOKENS = 16384
MOE_TOPK = 8
MOE_HIDDEN = 7168
MOE_FFN = 4096


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn_bf16(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """N(0, std^2) drawn in fp32 then rounded once to bf16."""
    x = torch.randn(shape, generator=generator(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ linear
def linear_small(device="cpu"):
    """X [256x512] and W [512x256], N(0,1) bf16, one generator seeded 0."""
    g = generator(0, device)
    X = torch.randn(256, 512, generator=g, device=device).to(torch.bfloat16)
    W = torch.randn(512, 256, generator=g, device=device).to(torch.bfloat16)
    return X, W


def dense_linear(M=8192, K=7168, N=18432, device="cpu"):
    """X [MxK] N(0,1) seed 0, W [KxN] N(0,0.02^2) seed 1, dY [MxN] N(0,1) seed 2."""
    X = randn_bf16((M, K), 0, device=device)
    W = randn_bf16((K, N), 1, std=0.02, device=device)
    dY = randn_bf16((M, N), 2, device=device)
    return X, W, dY


# ------------------------------------------------------------------ MXFP4
def qdq_small():
    """fp32 N(0,1) tensors of shapes (2,33), (3,17), (4,48,33), one generator seeded 0."""
    g = generator(0)
    return [torch.randn(s, generator=g, dtype=torch.float32) for s in ((2, 33), (3, 17), (4, 48, 33))]


def qdq_large(n: int = 8192, frac_rows: float = 0.01, device="cpu") -> torch.Tensor:
    """[n x n] fp32 N(0,1); round(frac*n) rows (randperm) times 2^u, u ~ U(-20,20).

    The factor 2^u is formed in fp64 and each product is rounded once to fp32.
    """
    g = generator(0)
    x = torch.randn(n, n, generator=g, dtype=torch.float32)
    k = int(round(frac_rows * n))
    rows = torch.randperm(n, generator=g)[:k]
    u = torch.rand(k, generator=g, dtype=torch.float64) * 40.0 - 20.0
    x[rows] = (x[rows].to(torch.float64) * torch.exp2(u)[:, None]).to(torch.float32)
    return x.to(device)


# ------------------------------------------------------------------ MoE
def moe_group_sizes(routing: str = "zipf_weights") -> list[int]:
    with open(MOE_SIZES_FILE if routing == "zipf_weights" else MOE_LAW_SIZES_FILE) as f:
        return list(json.load(f)["sizes"])


def group_end_from_sizes(sizes) -> torch.Tensor:
    """Cumulative group ends (int32), the layout the grouped entry points take."""
    return torch.tensor(np.cumsum(np.asarray(sizes, dtype=np.int64)), dtype=torch.int32)


def moe_routing(experts=MOE_EXPERTS, tokens=MOE_TOKENS, top_k=MOE_TOPK, seed=0,
                routing: str = "zipf_weights") -> torch.Tensor:
    """[tokens x top_k] expert ids: top-k distinct experts per token by
    multinomial sampling over expert weights -- i.i.d. Zipf(1.1) draws
    ("zipf_weights") or the Zipf law (e + 1)^-1.1 ("zipf_law")."""
    if routing == "zipf_weights":
        w = np.random.default_rng(seed).zipf(1.1, experts).astype(np.float64)
    elif routing == "zipf_law":
        w = (np.arange(experts, dtype=np.float64) + 1.0) ** -1.1
    else:
        raise ValueError(f"unknown routing {routing!r}; one of {ROUTINGS}")
    p = torch.tensor(w / w.sum(), dtype=torch.float64)
    return torch.multinomial(p.expand(tokens, experts), top_k, replacement=False,
                             generator=generator(seed))


def moe_row_tokens(idx: torch.Tensor, experts=MOE_EXPERTS) -> tuple[torch.Tensor, list[int]]:
    """Expert-ordered row -> token map and the per-expert sizes."""
    tok = torch.arange(idx.shape[0]).repeat_interleave(idx.shape[1])
    order = torch.argsort(idx.flatten(), stable=True)
    sizes = torch.bincount(idx.flatten(), minlength=experts).tolist()
    return tok[order], sizes


def moe_layer(device="cpu", with_dy=True, routing: str = "zipf_weights"):
    """X [131072x7168], W [32x7168x4096], dY [131072x4096] (bf16) and group_end [32]."""
    idx = moe_routing(routing=routing)
    row_tok, sizes = moe_row_tokens(idx)
    if sizes != moe_group_sizes(routing):
        raise RuntimeError("MoE routing draw differs from the frozen group sizes; "
                           "the random number streams of this torch build changed")
    xtok = randn_bf16((MOE_TOKENS, MOE_HIDDEN), 0, device=device)
    X = xtok.index_select(0, row_tok.to(device))
    del xtok
    W = randn_bf16((MOE_EXPERTS, MOE_HIDDEN, MOE_FFN), 1, std=0.02, device=device)
    dY = randn_bf16((X.shape[0], MOE_FFN), 2, device=device) if with_dy else None
    return X, W, dY, group_end_from_sizes(sizes)
