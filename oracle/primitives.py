"""fp64 definitions of the library's two standalone GEMM entry points.

TEST INFRASTRUCTURE ONLY (see the package docstring).

grouped_gemm: linear layer grouping runs several (input, weight) products
as one batched multiply (BOOST project page, "Three supporting changes";
the awesome-system-papers summary, batched GEMM over (input, weight) pairs).
The definition of the batch is simply each pair's product; the epilogues
are the elementwise steps the block fuses after them (residual add, the
SwiGLU of the MLP, a per-row scale).

The Online RMSNorm GEMM is ``block.online_rmsnorm_matmul``.
"""
from __future__ import annotations

import numpy as np

from .block import silu


def gemm(layout: str, X, W):
    """NT: X W^T (X [M,K], W [N,K]); NN: X W (W [K,N]); TN: X^T W (X [K,M])."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if layout == "NT":
        return X @ W.T
    if layout == "NN":
        return X @ W
    if layout == "TN":
        return X.T @ W
    raise ValueError(layout)


def grouped_gemm(layout: str, pairs, epilogue: str = "none", aux=None):
    """Products of every (X, W) pair, then the epilogue.

    epilogue: "none"; "residual" (+ aux, an [M, N] matrix); "row_scale"
    (row i divided by aux[i]); "swiglu" (two pairs -> SiLU(P0) * P1).
    """
    outs = [gemm(layout, X, W) for X, W in pairs]
    if epilogue == "none":
        return outs
    if epilogue == "residual":
        return [o + np.asarray(aux, dtype=np.float64) for o in outs]
    if epilogue == "row_scale":
        s = np.asarray(aux, dtype=np.float64)
        return [o / s[:, None] for o in outs]
    if epilogue == "swiglu":
        if len(outs) != 2:
            raise ValueError("SwiGLU takes two pairs")
        return [silu(outs[0]) * outs[1]]
    raise ValueError(epilogue)
