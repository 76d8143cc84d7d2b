"""One rank's GEMMs of the low-rank block under two tensor-parallel splits.

BOOST project page, "Move the chunk boundary to the bottleneck": standard
(vanilla) tensor parallelism treats each factor pair as one chunk, so the
down-projection A [r, d_in] is split along its r outputs and the
up-projection B [d_out, r] along its r inputs; every GEMM of a rank then
has an r / k wide side, and every chunk ends with an all-reduce of a full
d- or d_ff-wide activation. The bottleneck-aware split starts a chunk at an
up-projection split along its outputs (d / k or d_ff / k) and ends it at the
next down-projection split along its inputs, so r stays whole and the only
all-reduce per chunk is r wide (with the Online RMSNorm sum of squares for
the norm chunks). The page states the consequence for LLaMA-7B MLP blocks
as 2.5x the arithmetic intensity of the vanilla split.

This module lists, for one rank of k, the forward GEMMs of both splits
(M x N x K, operand pairs per launch) and their backward products (the
input gradient as an NN product, the weight gradient as a TN product with
fp32 output, K split over slices when its grid is small, as the block's own
weight gradients are), and times each through the library's entry points on
synthetic operands: the same kernels for both splits. Elementwise work
between the GEMMs (the vanilla split's SwiGLU after its d_ff-wide
all-reduce, norm backward, row dots) and the all-reduces themselves are
not run; the all-reduce volume per token is reported from the split.

Host-side plumbing only: operands are torch device tensors, every product
runs in the library.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import (LR_BF16, LR_EPI_NONE, LR_EPI_SWIGLU_PAIR, LR_LAYOUT_NN, LR_LAYOUT_NT,
               LR_LAYOUT_TN, grouped_lowrank_gemm, grouped_lowrank_gemm_workspace_bytes,
               online_rmsnorm_gemm)


@dataclasses.dataclass(frozen=True)
class Gemm:
    """A forward product Y_g = X_g W_g^T (g < G) of one rank: X [M, K], W [N, K]."""
    name: str
    mlp: bool          # part of the MLP block (for the MLP intensity figure)
    G: int             # operand pairs in one launch
    M: int
    N: int
    K: int
    norm: bool = False     # Online RMSNorm fused into the product (first pair)
    d_norm: int = 0        # RMS divisor of the norm (the global hidden width)
    partial: bool = False  # bottleneck split: the unscaled partial and its sum of squares
    swiglu: bool = False   # two pairs combined by SwiGLU in the epilogue

    def flops(self) -> float:
        return 2.0 * self.G * self.M * self.N * self.K


def vanilla_gemms(T: int, d: int, r: int, F: int, k: int) -> list[Gemm]:
    """Rank 0 of k under the per-factor-pair split: r / k wide products."""
    rk = r // k
    return [
        Gemm("QKV down (Online RMSNorm)", False, 1, T, 3 * rk, d, norm=True, d_norm=d),
        Gemm("QKV up", False, 3, T, d, rk),
        Gemm("O down", False, 1, T, rk, d),
        Gemm("O up", False, 1, T, d, rk),
        Gemm("gate/up down (Online RMSNorm)", True, 1, T, 2 * rk, d, norm=True, d_norm=d),
        Gemm("gate/up up", True, 2, T, F, rk),
        Gemm("down down", True, 1, T, rk, F),
        Gemm("down up", True, 1, T, d, rk),
    ]


def btp_gemms(T: int, d: int, r: int, F: int, k: int) -> list[Gemm]:
    """Rank 0 of k under the bottleneck-aware split: d / k and d_ff / k wide
    products with r whole; the norm chunks emit unscaled partials."""
    dk, Fk = d // k, F // k
    return [
        Gemm("QKV down (Online RMSNorm)", False, 1, T, 3 * r, dk, norm=True, d_norm=d,
             partial=True),
        Gemm("QKV up", False, 3, T, dk, r),
        Gemm("O down", False, 1, T, r, dk),
        Gemm("O up", False, 1, T, dk, r),
        Gemm("gate/up down (Online RMSNorm)", True, 1, T, 2 * r, dk, norm=True, d_norm=d,
             partial=True),
        Gemm("gate/up up + SwiGLU", True, 2, T, Fk, r, swiglu=True),
        Gemm("down down", True, 1, T, r, Fk),
        Gemm("down up", True, 1, T, dk, r),
    ]


def allreduce_values_per_token(split: str, d: int, r: int, F: int) -> int:
    """Values one rank sends per token per pass through the block (the page's
    volume table: 5d + 2d_ff for the vanilla split, 7r for BOOST)."""
    return 5 * d + 2 * F if split == "vanilla" else 7 * r


def products(g: Gemm) -> list[tuple[str, str, int, int, int, int]]:
    """(label, layout, G, M, N, K) of the forward product and its two backward
    products: dX = dY W (NN) and dW = dY^T X (TN, fp32)."""
    return [
        (g.name, "NT", g.G, g.M, g.N, g.K),
        (g.name + " dX", "NN", g.G, g.M, g.K, g.N),
        (g.name + " dW", "TN", g.G, g.N, g.K, g.M),
    ]


def work_bytes(layout: str, G: int, M: int, N: int, K: int, swiglu: bool = False) -> float:
    """Algorithmic bytes: bf16 operands read once, the output written once
    (fp32 for TN, one bf16 matrix for a SwiGLU pair)."""
    out = 4 if layout == "TN" else 2
    nout = 1 if swiglu else G
    return G * 2.0 * (M * K + N * K) + nout * out * M * N


class Operands:
    """Synthetic bf16 operands of one product, allocated once."""

    def __init__(self, layout: str, G: int, M: int, N: int, K: int, gen: torch.Generator,
                 device="cuda"):
        bf = torch.bfloat16

        def rnd(*shape, scale=1.0):
            return (torch.randn(*shape, generator=gen, device=device) * scale).to(bf)

        xs = (K, M) if layout == "TN" else (M, K)
        ws = (N, K) if layout == "NT" else (K, N)
        self.X = [rnd(*xs) for _ in range(G)]
        self.W = [rnd(*ws, scale=1.0 / np.sqrt(K)) for _ in range(G)]
        odt = torch.float32 if layout == "TN" else bf
        self.Y = [torch.empty(M, N, dtype=odt, device=device) for _ in range(G)]
        self.gamma = (1.0 + 0.1 * torch.randn(K, generator=gen, device=device)).to(bf)
        self.ss = torch.empty(M, dtype=torch.float32, device=device)
        self.rms = torch.empty(M, dtype=torch.float32, device=device)
        self.ws = None
        if layout == "TN":
            pairs = [dict(M=M, N=N, K=K, X=x, W=w, Y=y)
                     for x, w, y in zip(self.X, self.W, self.Y)]
            nb = grouped_lowrank_gemm_workspace_bytes(pairs, LR_BF16, LR_LAYOUT_TN)
            if nb:
                self.ws = torch.empty(nb, dtype=torch.uint8, device=device)


def run_product(layout: str, g: Gemm, ops: Operands, M: int, N: int, K: int) -> None:
    """One launch of a product through the library."""
    lay = {"NT": LR_LAYOUT_NT, "NN": LR_LAYOUT_NN, "TN": LR_LAYOUT_TN}[layout]
    if layout == "NT" and g.norm:
        online_rmsnorm_gemm(ops.X[0], ops.gamma, ops.W[0], ops.Y[0], n_panels=1,
                            d_norm=g.d_norm, eps=1e-5,
                            rms_out=None if g.partial else ops.rms,
                            ss_out=ops.ss, emit_partial=g.partial)
        return
    epi = LR_EPI_SWIGLU_PAIR if (layout == "NT" and g.swiglu) else LR_EPI_NONE
    pairs = [dict(M=M, N=N, K=K, X=x, W=w, Y=y) for x, w, y in zip(ops.X, ops.W, ops.Y)]
    grouped_lowrank_gemm(pairs, LR_BF16, lay, epi, ws=ops.ws)


def time_split(gemms: list[Gemm], reps: int = 5, seed: int = 0) -> list[dict]:
    """Time every product of a split (median of reps launches after one warm-up)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    rows = []
    for g in gemms:
        for label, layout, G, M, N, K in products(g):
            ops = Operands(layout, G, M, N, K, gen)
            run_product(layout, g, ops, M, N, K)
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                run_product(layout, g, ops, M, N, K)
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            ms = float(np.median(ts))
            fl = 2.0 * G * M * N * K
            by = work_bytes(layout, G, M, N, K, g.swiglu and layout == "NT")
            rows.append({"gemm": label, "mlp": g.mlp, "layout": layout, "G": G, "M": M, "N": N,
                         "K": K, "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                         "flop_per_byte": round(fl / by, 1), "flops": fl, "bytes": by})
            del ops
    torch.cuda.empty_cache()
    return rows


def summarize(rows: list[dict], peak_tflops: float) -> dict:
    def agg(sel):
        fl = sum(r["flops"] for r in sel)
        by = sum(r["bytes"] for r in sel)
        ms = sum(r["ms"] for r in sel)
        return {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / peak_tflops, 4),
                "flop_per_byte": round(fl / by, 1)}
    out = agg(rows)
    out["mlp"] = agg([r for r in rows if r["mlp"]])
    return out
