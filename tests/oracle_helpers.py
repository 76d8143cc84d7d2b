"""Helpers shared by the oracle tests: small seeded problems and a torch pin.

The torch pin builds the same block from torch's own fp64 library routines
(``rms_norm``, ``linear``, ``silu``) and differentiates it with autograd. It
shares no arithmetic with the numpy oracle, so agreement pins the oracle's
forward and its hand-written backward to independent implementations.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as Fn

import synth

W_NAMES = ("gamma1", "gamma2", "A_q", "A_k", "A_v", "B_q", "B_k", "B_v",
           "A_o", "B_o", "A_g", "A_u", "B_g", "B_u", "A_dn", "B_dn")


def small_problem(T=6, d=16, r=4, F=24, seed=0, D=None):
    s = synth.BlockShape("pin", T=T, d=d, r=r, F=F, D=D or d, dtype="f32", seed=seed)
    inp = synth.make_inputs(s)
    f64 = {k: v.astype(np.float64) for k, v in inp.items()}
    W = {k: f64[k] for k in W_NAMES}
    return s, W, f64


def torch_block(W, X, O, dY, dQ, dK, dV, eps, D=None):
    """fp64 torch forward + autograd backward of the block.

    When D exceeds the width d, the block is embedded in a width-D block
    whose other columns (of X, O, the upstream gradients and every weight
    slice) are zero; torch's rms_norm then normalises over D columns.
    Returns (forward dict, grad dict) restricted to the first d columns.
    """
    d = X.shape[1]
    D = D or d
    pad = D - d
    F_ = W["B_g"].shape[0]

    def t(a):
        return torch.tensor(a, dtype=torch.float64)

    def pad_cols(a):
        return np.pad(a, ((0, 0), (0, pad))) if pad else a

    def pad_rows(a):
        return np.pad(a, ((0, pad), (0, 0))) if pad else a

    P = {}
    for n in W_NAMES:
        a = W[n]
        if n.startswith("gamma"):
            a = np.pad(a, (0, pad), constant_values=1.0) if pad else a
        elif n in ("A_q", "A_k", "A_v", "A_o", "A_g", "A_u"):
            a = pad_cols(a)
        elif n in ("B_q", "B_k", "B_v", "B_o", "B_dn"):
            a = pad_rows(a)
        P[n] = t(a).requires_grad_(True)
    Xt = t(pad_cols(X)).requires_grad_(True)
    Ot = t(pad_cols(O)).requires_grad_(True)
    xn = Fn.rms_norm(Xt, (D,), weight=P["gamma1"], eps=eps)
    Q = Fn.linear(Fn.linear(xn, P["A_q"]), P["B_q"])
    K = Fn.linear(Fn.linear(xn, P["A_k"]), P["B_k"])
    V = Fn.linear(Fn.linear(xn, P["A_v"]), P["B_v"])
    h = Xt + Fn.linear(Fn.linear(Ot, P["A_o"]), P["B_o"])
    hn = Fn.rms_norm(h, (D,), weight=P["gamma2"], eps=eps)
    m = Fn.silu(Fn.linear(Fn.linear(hn, P["A_g"]), P["B_g"])) * \
        Fn.linear(Fn.linear(hn, P["A_u"]), P["B_u"])
    Y = h + Fn.linear(Fn.linear(m, P["A_dn"]), P["B_dn"])
    L = ((t(pad_cols(dY)) * Y).sum() + (t(pad_cols(dQ)) * Q).sum()
         + (t(pad_cols(dK)) * K).sum() + (t(pad_cols(dV)) * V).sum())
    L.backward()
    fwd = {"Q": Q, "K": K, "V": V, "Y": Y}
    fwd = {k: v.detach().numpy()[:, :d] for k, v in fwd.items()}
    G = {"X": Xt.grad.numpy()[:, :d], "O": Ot.grad.numpy()[:, :d]}
    for n in W_NAMES:
        g = P[n].grad.numpy()
        if n.startswith("gamma"):
            g = g[:d]
        elif n in ("A_q", "A_k", "A_v", "A_o", "A_g", "A_u"):
            g = g[:, :d]
        elif n in ("B_q", "B_k", "B_v", "B_o", "B_dn"):
            g = g[:d, :]
        G[n] = g
    assert F_ == G["B_g"].shape[0]
    return fwd, G


def rel_err(a, b):
    """max|a - b| / max|b|, the parity metric."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))
