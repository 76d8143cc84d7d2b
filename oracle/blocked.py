"""Full-workload driver of the oracle: row blocks, grouped output names.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The block is token-local except for the weight and gamma gradients, which
are sums over tokens. This driver runs the plain forward and backward of
``block.py`` on consecutive blocks of rows (to bound host memory at the full
16384-token workloads) and adds up the weight gradients block by block. That
splits each sum over tokens into partial sums; nothing else is reordered.

Outputs use the names and layouts the GPU library writes: the grouped
activations qkv_r = [q_r | k_r | v_r] and gu_r = [g_r | u_r], and the grouped
down-projection gradients dA_qkv = [dA_q; dA_k; dA_v], dA_gu = [dA_g; dA_u].
"""
from __future__ import annotations

import numpy as np

from .block import block_backward, block_forward, block_forward_online
from .share import share_forward

_WEIGHTS = ("gamma1", "gamma2", "A_q", "A_k", "A_v", "B_q", "B_k", "B_v",
            "A_o", "B_o", "A_g", "A_u", "B_g", "B_u", "A_dn", "B_dn")


def grouped_views(fwd):
    """qkv_r, gu_r from the separate r-wide activations."""
    return (np.concatenate([fwd["q_r"], fwd["k_r"], fwd["v_r"]], axis=1),
            np.concatenate([fwd["g_r"], fwd["u_r"]], axis=1))


def _accumulate(acc, grads):
    """Add one row block's weight and gamma gradients into the running sums.

    The gradients are sums over tokens (project page, "Three supporting
    changes": the weights see every token), so the blocks' parts add up."""
    for k, v in grads.items():
        acc[k] = v if k not in acc else acc[k] + v


def _weights64(inp):
    return {n: np.asarray(inp[n], dtype=np.float64) for n in _WEIGHTS}


def run_fwd_bwd(inp, *, D: int, eps: float, n_panels: int = 1,
                partials: bool = False, rows=None, row_block: int = 2048,
                backward: bool = True, weight_grads: bool = True,
                on_rows=None):
    """Forward and backward of the block on the seeded inputs ``inp``.

    inp        float32 arrays keyed as in ``synth.INPUT_ORDER`` (the exact
               values the GPU receives); widened to float64 here.
    D, eps     RMS divisor and epsilon.
    n_panels   Online RMSNorm K-panels; with P > 1 the forward also returns
               ss_panels1, ss_panels2 [P, T].
    partials   rank-share mode: the forward runs as a lone tensor-parallel
               rank and also returns P_qkv, ss1, P_gu, ss2.
    rows       optional row indices; the weight gradients need every row and
               are skipped when ``rows`` is given.
    on_rows    optional callback(row_indices, dict of row-local outputs);
               without it the row-local outputs are gathered and returned.

    Returns a dict with the row-local outputs (unless ``on_rows``) and, when
    computed, the weight and gamma gradients dgamma1 ... dB_dn (float64).
    """
    W = _weights64(inp)
    T = inp["X"].shape[0]
    idx = np.arange(T) if rows is None else np.asarray(rows)
    do_wgrad = backward and weight_grads and rows is None
    acc = {}
    gathered = {}
    for b0 in range(0, len(idx), row_block):
        sel = idx[b0:b0 + row_block]
        X = inp["X"][sel].astype(np.float64)
        O = inp["O"][sel].astype(np.float64)
        if partials:
            fwd = share_forward(W, X, O, D, eps)
        elif n_panels > 1:
            fwd = block_forward_online(W, X, O, D, eps, n_panels)
        else:
            fwd = block_forward(W, X, O, D, eps)
        qkv_r, gu_r = grouped_views(fwd)
        loc = dict(Q=fwd["Q"], K=fwd["K"], V=fwd["V"], Y=fwd["Y"], qkv_r=qkv_r,
                   o_r=fwd["o_r"], gu_r=gu_r, d_r=fwd["d_r"], rms1=fwd["rms1"],
                   rms2=fwd["rms2"])
        if n_panels > 1 and not partials:
            loc["ss_panels1"] = fwd["ss_panels1"].T   # gathered as [rows, P]
            loc["ss_panels2"] = fwd["ss_panels2"].T
        if partials:
            loc.update(P_qkv=fwd["P_qkv"], ss1=fwd["ss1"], P_gu=fwd["P_gu"],
                       ss2=fwd["ss2"])
        if backward:
            g = block_backward(W, X, O, fwd,
                               inp["dY"][sel].astype(np.float64),
                               inp["dQ"][sel].astype(np.float64),
                               inp["dK"][sel].astype(np.float64),
                               inp["dV"][sel].astype(np.float64), D, eps)
            loc["dX"], loc["dO"] = g["X"], g["O"]
            if do_wgrad:
                wg = dict(
                    dgamma1=g["gamma1"], dgamma2=g["gamma2"],
                    dA_qkv=np.concatenate([g["A_q"], g["A_k"], g["A_v"]], axis=0),
                    dB_q=g["B_q"], dB_k=g["B_k"], dB_v=g["B_v"],
                    dA_o=g["A_o"], dB_o=g["B_o"],
                    dA_gu=np.concatenate([g["A_g"], g["A_u"]], axis=0),
                    dB_g=g["B_g"], dB_u=g["B_u"], dA_dn=g["A_dn"], dB_dn=g["B_dn"])
                _accumulate(acc, wg)
        if on_rows is not None:
            on_rows(sel, loc)
        else:
            for k, v in loc.items():
                gathered.setdefault(k, []).append(v)
    out = {k: np.concatenate(v, axis=0) for k, v in gathered.items()}
    for k in ("ss_panels1", "ss_panels2"):
        if k in out:
            out[k] = np.ascontiguousarray(out[k].T)
    out.update(acc)
    return out
