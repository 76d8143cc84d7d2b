"""One tensor-parallel rank's share of the block under bottleneck-aware TP.

TEST INFRASTRUCTURE ONLY (see the package docstring).

BOOST project page, "Move the chunk boundary to the bottleneck": a chunk
starts at an up-projection split by columns (its output features) and ends at
the next down-projection split by rows (its input features), so the chunk's
only all-reduce carries an r-wide activation. Weights are split along d or
d_ff, never along r. Per block and pass the all-reduces carry 3r (Q,K,V),
r (O), 2r (gate, up) and r (down) values per token: 7r in total (the volume
table, "BOOST: 7bsr"). With Online RMSNorm ("Three supporting changes") the
two norm chunks also ship one sum of squares per token with their all-reduce.

Rank i of k holds columns S_i of the residual stream (d/k of them) and
columns S^F_i of the MLP (d_ff/k):
    gamma1, gamma2         -> gamma[S_i]
    A_q, A_k, A_v, A_o,
    A_g, A_u               -> A[:, S_i]     (input columns)
    B_q, B_k, B_v, B_o,
    B_dn                   -> B[S_i, :]     (output rows)
    B_g, B_u               -> B[S^F_i, :]
    A_dn                   -> A_dn[:, S^F_i]
    X, O, dY, dQ, dK, dV   -> [:, S_i]

The forward and backward are written as generators that yield each
all-reduce payload and receive the reduced value back, so the same code runs
as a lone rank whose all-reduce is the identity (the other ranks contribute
zero) and, in tests, as k ranks stepped in lock-step with a sum in between.

The backward uses, for the RMSNorm statistic sum_k(dxn * xn), the equal
r-wide dot sum_j(dz_r * z_r) with z_r = xn A^T and dxn = dz_r A: both r-wide
factors are replicated after the all-reduce, so the norm's backward needs no
collective of its own. This identity is algebra, not stated on the pages.
"""
from __future__ import annotations

import numpy as np

from .block import silu, silu_grad


def shard_weights(W, k: int, i: int):
    """Rank i's slices of the full weights W (see the module docstring)."""
    d = W["gamma1"].shape[0]
    F = W["B_g"].shape[0]
    if d % k or F % k:
        raise ValueError("d and d_ff must split evenly over the ranks")
    S = slice(i * d // k, (i + 1) * d // k)
    SF = slice(i * F // k, (i + 1) * F // k)
    Wi = {"gamma1": W["gamma1"][S], "gamma2": W["gamma2"][S]}
    for n in ("A_q", "A_k", "A_v", "A_o", "A_g", "A_u"):
        Wi[n] = W[n][:, S]
    for n in ("B_q", "B_k", "B_v", "B_o", "B_dn"):
        Wi[n] = W[n][S, :]
    for n in ("B_g", "B_u"):
        Wi[n] = W[n][SF, :]
    Wi["A_dn"] = W["A_dn"][:, SF]
    return Wi, S, SF


def norm_chunk_payload(gamma, x, A):
    """All-reduce payload of a norm chunk on one rank: the partial product of
    the gamma-scaled (not yet normalised) slice, (gamma * x) A^T, and the
    slice's per-row sum of squares (project page, "Three supporting changes",
    Online RMSNorm: the sum of squares travels with the chunk's all-reduce)."""
    return (gamma[None, :] * x) @ A.T, np.sum(x * x, axis=1)


def _forward_steps(Wi, Xi, Oi, D: int, eps: float):
    r = Wi["A_q"].shape[0]
    A_qkv = np.concatenate([Wi["A_q"], Wi["A_k"], Wi["A_v"]], axis=0)
    A_gu = np.concatenate([Wi["A_g"], Wi["A_u"]], axis=0)
    out = {}
    # Chunk ending at the grouped QKV down-projection: partial product of the
    # un-normalised (gamma-scaled) slice plus the slice's sum of squares.
    P_qkv, ss1 = norm_chunk_payload(Wi["gamma1"], Xi, A_qkv)
    out["P_qkv"], out["ss1"] = P_qkv, ss1
    P_qkv_red, ss1_red = yield (P_qkv, ss1)
    rms1 = np.sqrt(ss1_red / D + eps)
    qkv_r = P_qkv_red / rms1[:, None]
    q_r, k_r, v_r = qkv_r[:, :r], qkv_r[:, r:2 * r], qkv_r[:, 2 * r:]
    # Chunk from the QKV up-projections through attention to A_o.
    out["Q"] = q_r @ Wi["B_q"].T
    out["K"] = k_r @ Wi["B_k"].T
    out["V"] = v_r @ Wi["B_v"].T
    P_o = Oi @ Wi["A_o"].T
    (o_r,) = yield (P_o,)
    # Chunk from B_o through the residual and Online RMSNorm to A_gu.
    h = Xi + o_r @ Wi["B_o"].T
    P_gu, ss2 = norm_chunk_payload(Wi["gamma2"], h, A_gu)
    out["P_gu"], out["ss2"] = P_gu, ss2
    P_gu_red, ss2_red = yield (P_gu, ss2)
    rms2 = np.sqrt(ss2_red / D + eps)
    gu_r = P_gu_red / rms2[:, None]
    g_r, u_r = gu_r[:, :r], gu_r[:, r:]
    # Chunk from B_g, B_u through SwiGLU to A_dn.
    m = silu(g_r @ Wi["B_g"].T) * (u_r @ Wi["B_u"].T)
    P_dn = m @ Wi["A_dn"].T
    (d_r,) = yield (P_dn,)
    # Start of the next block's first chunk: B_dn and the residual.
    out["Y"] = h + d_r @ Wi["B_dn"].T
    out.update(q_r=q_r, k_r=k_r, v_r=v_r, o_r=o_r, g_r=g_r, u_r=u_r, d_r=d_r,
               rms1=rms1, rms2=rms2)
    return out


def _backward_steps(Wi, Xi, Oi, saved, dYi, dQi, dKi, dVi, D: int):
    r = Wi["A_q"].shape[0]
    q_r, k_r, v_r = saved["q_r"], saved["k_r"], saved["v_r"]
    o_r, g_r, u_r, d_r = saved["o_r"], saved["g_r"], saved["u_r"], saved["d_r"]
    s1, s2 = 1.0 / saved["rms1"], 1.0 / saved["rms2"]
    G = {}
    # Recompute the chunk-local d-wide tensors from the r-wide ones.
    h = Xi + o_r @ Wi["B_o"].T
    g = g_r @ Wi["B_g"].T
    u = u_r @ Wi["B_u"].T
    m = silu(g) * u
    # Y = h + d_r B_dn^T
    G["B_dn"] = dYi.T @ d_r
    (dd_r,) = yield (dYi @ Wi["B_dn"],)
    G["A_dn"] = dd_r.T @ m
    dm = dd_r @ Wi["A_dn"]
    dg = dm * u * silu_grad(g)
    du = dm * silu(g)
    G["B_g"] = dg.T @ g_r
    G["B_u"] = du.T @ u_r
    (dgu_r,) = yield (np.concatenate([dg @ Wi["B_g"], du @ Wi["B_u"]], axis=1),)
    # RMSNorm-2 backward with the r-wide statistic.
    gu_r = np.concatenate([g_r, u_r], axis=1)
    A_gu = np.concatenate([Wi["A_g"], Wi["A_u"]], axis=0)
    hn = Wi["gamma2"][None, :] * h * s2[:, None]
    dhn = dgu_r @ A_gu
    c2 = np.sum(dgu_r * gu_r, axis=1)
    G["A_g"] = dgu_r[:, :r].T @ hn
    G["A_u"] = dgu_r[:, r:].T @ hn
    G["gamma2"] = np.sum(dhn * h * s2[:, None], axis=0)
    dh = (dYi + s2[:, None] * Wi["gamma2"][None, :] * dhn
          - ((s2 * s2 / D) * c2)[:, None] * h)
    # h = X + o_r B_o^T
    G["B_o"] = dh.T @ o_r
    (do_r,) = yield (dh @ Wi["B_o"],)
    G["A_o"] = do_r.T @ Oi
    G["O"] = do_r @ Wi["A_o"]
    # Q, K, V up-projections.
    G["B_q"] = dQi.T @ q_r
    G["B_k"] = dKi.T @ k_r
    G["B_v"] = dVi.T @ v_r
    (dqkv_r,) = yield (np.concatenate(
        [dQi @ Wi["B_q"], dKi @ Wi["B_k"], dVi @ Wi["B_v"]], axis=1),)
    # RMSNorm-1 backward with the r-wide statistic.
    qkv_r = np.concatenate([q_r, k_r, v_r], axis=1)
    A_qkv = np.concatenate([Wi["A_q"], Wi["A_k"], Wi["A_v"]], axis=0)
    xn = Wi["gamma1"][None, :] * Xi * s1[:, None]
    dxn = dqkv_r @ A_qkv
    c1 = np.sum(dqkv_r * qkv_r, axis=1)
    G["A_q"] = dqkv_r[:, :r].T @ xn
    G["A_k"] = dqkv_r[:, r:2 * r].T @ xn
    G["A_v"] = dqkv_r[:, 2 * r:].T @ xn
    G["gamma1"] = np.sum(dxn * Xi * s1[:, None], axis=0)
    G["X"] = (dh + s1[:, None] * Wi["gamma1"][None, :] * dxn
              - ((s1 * s1 / D) * c1)[:, None] * Xi)
    return G


def _run_alone(gen):
    """Drive one rank whose all-reduce is the identity."""
    try:
        payload = next(gen)
        while True:
            payload = gen.send(payload)
    except StopIteration as stop:
        return stop.value


def _run_lockstep(gens):
    """Drive k ranks together; every all-reduce is a sum over the ranks."""
    payloads = [next(g) for g in gens]
    results = [None] * len(gens)
    while True:
        reduced = tuple(sum(p[j] for p in payloads) for j in range(len(payloads[0])))
        nxt = []
        for idx, g in enumerate(gens):
            try:
                nxt.append(g.send(reduced))
            except StopIteration as stop:
                results[idx] = stop.value
                nxt.append(None)
        if all(x is None for x in nxt):
            return results
        if any(x is None for x in nxt):
            raise RuntimeError("ranks disagree on the number of all-reduces")
        payloads = nxt


def share_forward(Wi, Xi, Oi, D: int, eps: float):
    """A lone rank's forward (identity all-reduce), with its partial sums.

    Returns Q, K, V, Y (this rank's d-columns), the r-wide activations,
    rms1, rms2 and the all-reduce payloads of the two norm chunks before
    reduction: P_qkv = (gamma1 * X) A_qkv^T, ss1 = sum X^2, P_gu, ss2. The
    payloads of the other two chunks are o_r and d_r themselves.
    """
    return _run_alone(_forward_steps(Wi, Xi, Oi, D, eps))


def share_backward(Wi, Xi, Oi, saved, dYi, dQi, dKi, dVi, D: int):
    """A lone rank's backward (identity all-reduce) from the r-wide saves."""
    return _run_alone(_backward_steps(Wi, Xi, Oi, saved, dYi, dQi, dKi, dVi, D))


def simulate_tp_forward(W, X, O, k: int, D: int, eps: float):
    """k ranks in lock-step; returns the per-rank outputs and the slices."""
    parts = [shard_weights(W, k, i) for i in range(k)]
    gens = [_forward_steps(Wi, X[:, S], O[:, S], D, eps) for Wi, S, _ in parts]
    return _run_lockstep(gens), parts


def simulate_tp_backward(W, X, O, saved, dY, dQ, dK, dV, k: int, D: int):
    """k ranks' backward in lock-step from the (replicated) r-wide saves."""
    parts = [shard_weights(W, k, i) for i in range(k)]
    gens = [_backward_steps(Wi, X[:, S], O[:, S], saved, dY[:, S], dQ[:, S],
                            dK[:, S], dV[:, S], D) for Wi, S, _ in parts]
    return _run_lockstep(gens), parts
