"""Plain fp64 forward and backward of one low-rank LLaMA-2-style block.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The block (BOOST project page, "Move the chunk boundary to the bottleneck",
the decoder-block figure): every linear layer is a down-projection A [r, in]
followed by an up-projection B [out, r]; nothing sits between the two factors
(the SVD-style pair, "Larger batches and other bottleneck models"). Weights
are stored [out, in], so a layer computes y = x @ W.T.

    rms1 = sqrt(sum_k X^2 / D + eps);   xn = gamma1 * X / rms1
    q_r, k_r, v_r = xn A_q^T, xn A_k^T, xn A_v^T
    Q, K, V = q_r B_q^T, k_r B_k^T, v_r B_v^T         (to the attention core)
    o_r = O A_o^T                                      (O from the attention core)
    h = X + o_r B_o^T
    rms2 = sqrt(sum_k h^2 / D + eps);   hn = gamma2 * h / rms2
    g_r, u_r = hn A_g^T, hn A_u^T
    g, u = g_r B_g^T, u_r B_u^T;        m = SiLU(g) * u
    d_r = m A_dn^T
    Y = h + d_r B_dn^T

Readings taken where the pages are silent:
  * RMSNorm is gamma * x / sqrt(mean(x^2) + eps): no mean subtraction, no
    bias; eps = 1e-5 inside the square root (the pages give no value).
  * D, the divisor of the mean, is the global hidden width; it differs from
    the width this GPU holds only for a tensor-parallel rank share.
  * SwiGLU is SiLU(gate) * up with SiLU(z) = z / (1 + exp(-z)); the SiLU is
    on the gate projection ("gate and up projections", "Three supporting
    changes").
  * The attention core is outside the stack: O is an input, and dQ, dK, dV
    are inputs of the backward.

The backward differentiates L = <dY,Y> + <dQ,Q> + <dK,K> + <dV,V>.
"""
from __future__ import annotations

import numpy as np

GRAD_NAMES = (
    "X", "O", "gamma1", "gamma2",
    "A_q", "A_k", "A_v", "B_q", "B_k", "B_v",
    "A_o", "B_o", "A_g", "A_u", "B_g", "B_u", "A_dn", "B_dn",
)


# --------------------------------------------------------------------------
# Elementwise pieces
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d SiLU / dz = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


# --------------------------------------------------------------------------
# RMSNorm and Online RMSNorm
# --------------------------------------------------------------------------
def rms(x: np.ndarray, D: int, eps: float) -> np.ndarray:
    """Per-row root mean square: sqrt(sum_k x^2 / D + eps), shape [T]."""
    return np.sqrt(np.sum(x * x, axis=1) / D + eps)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, D: int, eps: float):
    """gamma * x / rms(x). Returns (normalised x, rms)."""
    r = rms(x, D, eps)
    return gamma[None, :] * x / r[:, None], r


def online_rmsnorm_matmul(x, gamma, A, n_panels: int, D: int, eps: float):
    """RMSNorm(x) @ A.T computed panel by panel, as Online RMSNorm does.

    BOOST project page, "Three supporting changes" (Online RMSNorm): each
    holder of a slice of the hidden vector normalises with its own local RMS,
    scales the output of its matmul back, and ships its sum of squares with
    the partial result; dividing by the global RMS then gives the exact
    normalised product. The awesome-system-papers summary names the per-row
    correction alpha = RMS_local / RMS_global.

    The hidden dimension is cut into ``n_panels`` contiguous panels of equal
    width w. For panel p with columns S_p:
        ss_p    = sum_{k in S_p} x_k^2
        rms_p   = sqrt(ss_p / w + eps)              (local RMS of the panel)
        Z_p     = ((gamma_p * x_p) / rms_p) @ A_p.T  (normalised locally)
        rms_g   = sqrt(sum_p ss_p / D + eps)        (global RMS)
        out     = sum_p (rms_p / rms_g) * Z_p        (alpha_p = rms_p / rms_g)

    Returns (out, rms_g, ss_panels[P, T]).
    """
    T, d = x.shape
    if d % n_panels:
        raise ValueError("hidden width must split into equal panels")
    w = d // n_panels
    ss, Z, loc = [], [], []
    for p in range(n_panels):
        cols = slice(p * w, (p + 1) * w)
        xp = x[:, cols]
        ss_p = np.sum(xp * xp, axis=1)
        rms_p = np.sqrt(ss_p / w + eps)
        Z_p = ((gamma[None, cols] * xp) / rms_p[:, None]) @ A[:, cols].T
        ss.append(ss_p)
        loc.append(rms_p)
        Z.append(Z_p)
    ss_tot = np.zeros(T)
    for ss_p in ss:
        ss_tot = ss_tot + ss_p
    rms_g = np.sqrt(ss_tot / D + eps)
    out = np.zeros((T, A.shape[0]))
    for rms_p, Z_p in zip(loc, Z):
        out = out + (rms_p / rms_g)[:, None] * Z_p
    return out, rms_g, np.stack(ss)


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------
def _up(z_r, B):
    return z_r @ B.T


def _recompute_h(W, X, o_r):
    return X + o_r @ W["B_o"].T


def _recompute_mlp(W, g_r, u_r):
    g = g_r @ W["B_g"].T
    u = u_r @ W["B_u"].T
    return g, u, silu(g) * u


def block_forward(W, X, O, D: int, eps: float, tape: bool = False):
    """Plain forward of the block (the definition in the module docstring).

    Returns a dict with Q, K, V, Y, the r-wide activations q_r, k_r, v_r,
    o_r, g_r, u_r, d_r and the row statistics rms1, rms2. With ``tape`` it
    also returns the d-wide intermediates xn, h, hn, g, u, m.
    """
    xn, rms1 = rmsnorm(X, W["gamma1"], D, eps)
    q_r = xn @ W["A_q"].T
    k_r = xn @ W["A_k"].T
    v_r = xn @ W["A_v"].T
    Q, K, V = _up(q_r, W["B_q"]), _up(k_r, W["B_k"]), _up(v_r, W["B_v"])
    o_r = O @ W["A_o"].T
    h = _recompute_h(W, X, o_r)
    hn, rms2 = rmsnorm(h, W["gamma2"], D, eps)
    g_r = hn @ W["A_g"].T
    u_r = hn @ W["A_u"].T
    g, u, m = _recompute_mlp(W, g_r, u_r)
    d_r = m @ W["A_dn"].T
    Y = h + d_r @ W["B_dn"].T
    out = dict(Q=Q, K=K, V=V, Y=Y, q_r=q_r, k_r=k_r, v_r=v_r, o_r=o_r,
               g_r=g_r, u_r=u_r, d_r=d_r, rms1=rms1, rms2=rms2)
    if tape:
        out.update(xn=xn, h=h, hn=hn, g=g, u=u, m=m)
    return out


def block_forward_online(W, X, O, D: int, eps: float, n_panels: int):
    """Forward with both norm + down-projection steps in the panel form.

    Same block as ``block_forward``; the two RMSNorm -> down-projection steps
    go through ``online_rmsnorm_matmul`` over ``n_panels`` K-panels with the
    grouped weights [A_q; A_k; A_v] and [A_g; A_u]. Also returns the per-panel
    sums of squares ss_panels1, ss_panels2 [P, T].
    """
    r = W["A_q"].shape[0]
    A_qkv = np.concatenate([W["A_q"], W["A_k"], W["A_v"]], axis=0)
    A_gu = np.concatenate([W["A_g"], W["A_u"]], axis=0)
    qkv_r, rms1, ssp1 = online_rmsnorm_matmul(X, W["gamma1"], A_qkv, n_panels, D, eps)
    q_r, k_r, v_r = qkv_r[:, :r], qkv_r[:, r:2 * r], qkv_r[:, 2 * r:]
    Q, K, V = _up(q_r, W["B_q"]), _up(k_r, W["B_k"]), _up(v_r, W["B_v"])
    o_r = O @ W["A_o"].T
    h = _recompute_h(W, X, o_r)
    gu_r, rms2, ssp2 = online_rmsnorm_matmul(h, W["gamma2"], A_gu, n_panels, D, eps)
    g_r, u_r = gu_r[:, :r], gu_r[:, r:]
    g, u, m = _recompute_mlp(W, g_r, u_r)
    d_r = m @ W["A_dn"].T
    Y = h + d_r @ W["B_dn"].T
    return dict(Q=Q, K=K, V=V, Y=Y, q_r=q_r, k_r=k_r, v_r=v_r, o_r=o_r,
                g_r=g_r, u_r=u_r, d_r=d_r, rms1=rms1, rms2=rms2,
                ss_panels1=ssp1, ss_panels2=ssp2)


def block_forward_grouped(W, X, O, D: int, eps: float):
    """Forward with linear layer grouping.

    BOOST project page, "Three supporting changes" (Linear layer grouping):
    the Q, K and V down-projections share their input and run as one matmul
    against the stacked weight [A_q; A_k; A_v] (width 3r); their three
    up-projections, which have different inputs, run as one batched matmul
    over (input, weight) pairs; gate and up are grouped the same way.
    """
    r = W["A_q"].shape[0]
    xn, rms1 = rmsnorm(X, W["gamma1"], D, eps)
    qkv_r = xn @ np.concatenate([W["A_q"], W["A_k"], W["A_v"]], axis=0).T
    ins = np.stack([qkv_r[:, :r], qkv_r[:, r:2 * r], qkv_r[:, 2 * r:]])
    wts = np.stack([W["B_q"], W["B_k"], W["B_v"]])
    QKV = np.matmul(ins, np.transpose(wts, (0, 2, 1)))
    o_r = O @ W["A_o"].T
    h = X + o_r @ W["B_o"].T
    hn, rms2 = rmsnorm(h, W["gamma2"], D, eps)
    gu_r = hn @ np.concatenate([W["A_g"], W["A_u"]], axis=0).T
    gu = np.matmul(np.stack([gu_r[:, :r], gu_r[:, r:]]),
                   np.transpose(np.stack([W["B_g"], W["B_u"]]), (0, 2, 1)))
    m = silu(gu[0]) * gu[1]
    d_r = m @ W["A_dn"].T
    Y = h + d_r @ W["B_dn"].T
    return dict(Q=QKV[0], K=QKV[1], V=QKV[2], Y=Y, q_r=ins[0], k_r=ins[1],
                v_r=ins[2], o_r=o_r, g_r=gu_r[:, :r], u_r=gu_r[:, r:], d_r=d_r,
                rms1=rms1, rms2=rms2)


def block_loss(W, X, O, dY, dQ, dK, dV, D: int, eps: float) -> float:
    """L = <dY,Y> + <dQ,Q> + <dK,K> + <dV,V>, the scalar the backward differentiates."""
    f = block_forward(W, X, O, D, eps)
    return float(np.sum(dY * f["Y"]) + np.sum(dQ * f["Q"])
                 + np.sum(dK * f["K"]) + np.sum(dV * f["V"]))


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------
def _rmsnorm_backward(x, gamma, r, dxn, D: int):
    """Backward of xn = gamma * x / r with r = sqrt(sum x^2 / D + eps).

    With s = 1/r:  dx = s * gamma * dxn - (s^2 / D) * x * sum_k(dxn * xn)
                   dgamma = sum_t dxn * x * s
    """
    s = 1.0 / r
    xn = gamma[None, :] * x * s[:, None]
    c = np.sum(dxn * xn, axis=1)
    dx = s[:, None] * gamma[None, :] * dxn - ((s * s / D) * c)[:, None] * x
    dgamma = np.sum(dxn * x * s[:, None], axis=0)
    return dx, dgamma


def block_backward_tape(W, t, X, O, dY, dQ, dK, dV, D: int):
    """Backward from a full tape (every intermediate of the forward stored).

    ``t`` holds q_r, k_r, v_r, o_r, g_r, u_r, d_r, rms1, rms2, xn, h, hn,
    g, u, m. Returns the gradient of every input, weight and gamma.
    """
    G = {}
    # Y = h + d_r B_dn^T
    G["B_dn"] = dY.T @ t["d_r"]
    dd_r = dY @ W["B_dn"]
    dh = dY.copy()
    # d_r = m A_dn^T
    G["A_dn"] = dd_r.T @ t["m"]
    dm = dd_r @ W["A_dn"]
    # m = SiLU(g) * u
    dg = dm * t["u"] * silu_grad(t["g"])
    du = dm * silu(t["g"])
    # g = g_r B_g^T, u = u_r B_u^T
    G["B_g"] = dg.T @ t["g_r"]
    G["B_u"] = du.T @ t["u_r"]
    dg_r = dg @ W["B_g"]
    du_r = du @ W["B_u"]
    # g_r = hn A_g^T, u_r = hn A_u^T
    G["A_g"] = dg_r.T @ t["hn"]
    G["A_u"] = du_r.T @ t["hn"]
    dhn = dg_r @ W["A_g"] + du_r @ W["A_u"]
    # hn = RMSNorm(h)
    dh_n, G["gamma2"] = _rmsnorm_backward(t["h"], W["gamma2"], t["rms2"], dhn, D)
    dh = dh + dh_n
    # h = X + o_r B_o^T
    dX = dh.copy()
    G["B_o"] = dh.T @ t["o_r"]
    do_r = dh @ W["B_o"]
    # o_r = O A_o^T
    G["A_o"] = do_r.T @ O
    G["O"] = do_r @ W["A_o"]
    # Q = q_r B_q^T (and K, V)
    G["B_q"] = dQ.T @ t["q_r"]
    G["B_k"] = dK.T @ t["k_r"]
    G["B_v"] = dV.T @ t["v_r"]
    dq_r = dQ @ W["B_q"]
    dk_r = dK @ W["B_k"]
    dv_r = dV @ W["B_v"]
    # q_r = xn A_q^T (and k, v)
    G["A_q"] = dq_r.T @ t["xn"]
    G["A_k"] = dk_r.T @ t["xn"]
    G["A_v"] = dv_r.T @ t["xn"]
    dxn = dq_r @ W["A_q"] + dk_r @ W["A_k"] + dv_r @ W["A_v"]
    # xn = RMSNorm(X)
    dX_n, G["gamma1"] = _rmsnorm_backward(X, W["gamma1"], t["rms1"], dxn, D)
    G["X"] = dX + dX_n
    return G


def block_backward(W, X, O, saved, dY, dQ, dK, dV, D: int, eps: float):
    """Backward that keeps only the r-wide activations and recomputes the rest.

    BOOST project page, "Three supporting changes" (Checkpointing without
    communication): only the r-wide activations at the chunk boundaries are
    stored; the backward recomputes each chunk from them. ``saved`` holds
    q_r, k_r, v_r, o_r, g_r, u_r, d_r (7r values per token) and rms1, rms2;
    X and O are the caller's inputs, re-read. The d-wide tensors xn, h, hn,
    g, u, m are recomputed with the same expressions as the forward, then the
    tape backward runs.
    """
    t = {k: saved[k] for k in ("q_r", "k_r", "v_r", "o_r", "g_r", "u_r", "d_r",
                               "rms1", "rms2")}
    t["xn"] = W["gamma1"][None, :] * X / t["rms1"][:, None]
    t["h"] = _recompute_h(W, X, t["o_r"])
    t["hn"] = W["gamma2"][None, :] * t["h"] / t["rms2"][:, None]
    t["g"], t["u"], t["m"] = _recompute_mlp(W, t["g_r"], t["u_r"])
    del eps  # the saved rms already contains it
    return block_backward_tape(W, t, X, O, dY, dQ, dK, dV, D)
