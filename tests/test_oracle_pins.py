"""Pins of the fp64 oracle against things other than itself.

Each test names what fixes the expected value: a closed form, torch's own
library routines with autograd, finite differences of the oracle's forward,
or an exactness statement of the BOOST pages turned into an identity.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle import block as ob
from oracle import share as osh
from tests.oracle_helpers import W_NAMES, rel_err, small_problem, torch_block

EPS = 1e-5


# ---------------------------------------------------------------- closed forms
def test_silu_closed_form():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    v = ob.silu(z)
    assert v[0] == 0.0
    assert v[1] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert v[2] == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert v[3] == pytest.approx(40.0, rel=1e-15)
    assert abs(v[4]) < 1e-15
    g = ob.silu_grad(z)
    assert g[0] == pytest.approx(0.5, rel=1e-15)          # sigmoid(0) = 1/2
    assert g[3] == pytest.approx(1.0, rel=1e-12)
    # derivative against a central difference of the closed form
    zz = np.linspace(-6, 6, 25)
    h = 1e-6
    fd = (ob.silu(zz + h) - ob.silu(zz - h)) / (2 * h)
    assert np.max(np.abs(fd - ob.silu_grad(zz))) < 1e-8


def test_rmsnorm_closed_forms():
    # constant row c: rms = sqrt(c^2 + eps), output gamma * c / sqrt(c^2 + eps)
    x = np.full((3, 8), 2.0)
    x[1] = -0.5
    x[2] = 0.0
    gamma = np.linspace(0.5, 1.5, 8)
    y, r = ob.rmsnorm(x, gamma, 8, EPS)
    for i, c in enumerate((2.0, -0.5, 0.0)):
        assert r[i] == pytest.approx(math.sqrt(c * c + EPS), rel=1e-15)
        assert np.allclose(y[i], gamma * c / math.sqrt(c * c + EPS), rtol=1e-15, atol=0)
    # gamma = 1, eps = 0: every output row has unit mean square
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 32))
    y, _ = ob.rmsnorm(x, np.ones(32), 32, 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-14)
    # divisor D: a row padded with zeros to width D normalises the same way
    y1, _ = ob.rmsnorm(x, np.ones(32), 128, 0.0)
    y2, _ = ob.rmsnorm(np.pad(x, ((0, 0), (0, 96))), np.ones(128), 128, 0.0)
    assert np.allclose(y1, y2[:, :32], rtol=1e-14)


# ----------------------------------------------------------- torch library pin
@pytest.mark.parametrize("shape", [dict(T=6, d=16, r=4, F=24),
                                   dict(T=9, d=24, r=8, F=40, seed=5)])
def test_forward_and_backward_match_torch_autograd(shape):
    s, W, f = small_problem(**shape)
    fwd = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    G = ob.block_backward(W, f["X"], f["O"], fwd, f["dY"], f["dQ"], f["dK"],
                          f["dV"], s.D, EPS)
    tf, tg = torch_block(W, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"], EPS)
    for k in ("Q", "K", "V", "Y"):
        assert rel_err(fwd[k], tf[k]) < 1e-13, k
    for k in ("X", "O") + W_NAMES:
        assert rel_err(G[k], tg[k]) < 1e-12, k


def test_rank_share_divisor_matches_zero_padded_torch_block():
    """A lone rank (identity all-reduce) = the width-D block with zero peers."""
    s, W, f = small_problem(T=5, d=12, r=6, F=20, D=48, seed=7)
    fwd = osh.share_forward(W, f["X"], f["O"], s.D, EPS)
    G = osh.share_backward(W, f["X"], f["O"], fwd, f["dY"], f["dQ"], f["dK"],
                           f["dV"], s.D)
    tf, tg = torch_block(W, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"],
                         EPS, D=s.D)
    for k in ("Q", "K", "V", "Y"):
        assert rel_err(fwd[k], tf[k]) < 1e-13, k
    for k in ("X", "O") + W_NAMES:
        assert rel_err(G[k], tg[k]) < 1e-12, k
    # and the plain block with the divisor D agrees with the share
    pf = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    pg = ob.block_backward(W, f["X"], f["O"], pf, f["dY"], f["dQ"], f["dK"],
                           f["dV"], s.D, EPS)
    for k in ("Y", "Q"):
        assert rel_err(pf[k], tf[k]) < 1e-13
    for k in ("X", "gamma1", "A_q"):
        assert rel_err(pg[k], tg[k]) < 1e-12


# --------------------------------------------------------- finite differences
def _loss_fn(form, n_panels):
    def L(W, X, O, dY, dQ, dK, dV, D):
        if form == "plain":
            y = ob.block_forward(W, X, O, D, EPS)
        else:
            y = ob.block_forward_online(W, X, O, D, EPS, n_panels)
        return (np.sum(dY * y["Y"]) + np.sum(dQ * y["Q"]) + np.sum(dK * y["K"])
                + np.sum(dV * y["V"]))
    return L


@pytest.mark.parametrize("form,n_panels", [("plain", 1), ("online", 1), ("online", 2)])
def test_finite_differences_every_coordinate(form, n_panels):
    """Central differences (h = 1e-6) of L for every input coordinate."""
    s, W, f = small_problem(T=4, d=8, r=2, F=12, seed=11)
    L = _loss_fn(form, n_panels)
    fwd = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    G = ob.block_backward(W, f["X"], f["O"], fwd, f["dY"], f["dQ"], f["dK"],
                          f["dV"], s.D, EPS)
    args = dict(W=W, X=f["X"], O=f["O"])
    h = 1e-6
    worst = 0.0
    for name in ("X", "O") + W_NAMES:
        tgt = args["W"][name] if name in W else args[name]
        it = np.nditer(tgt, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = tgt[ix]
            tgt[ix] = old + h
            lp = L(W, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"], s.D)
            tgt[ix] = old - h
            lm = L(W, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"], s.D)
            tgt[ix] = old
            fd = (lp - lm) / (2 * h)
            an = G[name][ix]
            err = abs(fd - an) / max(1.0, abs(an))
            worst = max(worst, err)
            assert err < 1e-6, (name, ix, fd, an)
    assert worst < 1e-6


def test_finite_differences_sampled_tiny_config_shape():
    """20 random coordinates per tensor at the tiny workload's shapes."""
    s, W, f = small_problem(T=16, d=256, r=64, F=688, seed=0)
    fwd = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    G = ob.block_backward(W, f["X"], f["O"], fwd, f["dY"], f["dQ"], f["dK"],
                          f["dV"], s.D, EPS)
    L = _loss_fn("plain", 1)
    rng = np.random.default_rng(1)
    h = 1e-5
    for name in ("X", "O") + W_NAMES:
        tgt = W[name] if name in W else f[name]
        for _ in range(20):
            ix = tuple(int(rng.integers(0, n)) for n in tgt.shape)
            old = tgt[ix]
            tgt[ix] = old + h
            lp = L(W, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"], s.D)
            tgt[ix] = old - h
            lm = L(W, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"], s.D)
            tgt[ix] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - G[name][ix]) <= 1e-6 * max(1.0, abs(G[name][ix])), (name, ix)


# ------------------------------------------------ exactness claims as identities
@pytest.mark.parametrize("P", [1, 2, 4])
def test_online_rmsnorm_panel_form_is_exact(P):
    """Online RMSNorm gives the exact normalised product (project page,
    'Three supporting changes'; alpha correction per row, summary page)."""
    rng = np.random.default_rng(P)
    T, d, N = 33, 64, 12
    x = rng.standard_normal((T, d)) * rng.uniform(0.1, 10.0, (T, 1))
    x[3, : d // P] = 0.0            # a panel that is all zeros
    gamma = 1 + 0.1 * rng.standard_normal(d)
    A = rng.standard_normal((N, d)) / 8
    out, rms_g, ssp = ob.online_rmsnorm_matmul(x, gamma, A, P, d, EPS)
    xn, r = ob.rmsnorm(x, gamma, d, EPS)
    ref = xn @ A.T
    assert rel_err(out, ref) < 1e-12
    assert np.allclose(rms_g, r, rtol=1e-14)
    assert ssp.shape == (P, T)
    assert np.allclose(ssp.sum(axis=0), np.sum(x * x, axis=1), rtol=1e-13)
    # the per-panel sums are sums over contiguous panels
    w = d // P
    assert np.allclose(ssp[1 % P], np.sum(x[:, (1 % P) * w:((1 % P) + 1) * w] ** 2, axis=1))


def test_online_forward_equals_plain_forward():
    s, W, f = small_problem(T=7, d=32, r=8, F=40, seed=2)
    a = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    for P in (1, 2, 4):
        b = ob.block_forward_online(W, f["X"], f["O"], s.D, EPS, P)
        for k in ("Q", "K", "V", "Y", "q_r", "g_r", "d_r", "rms1", "rms2"):
            assert rel_err(b[k], a[k]) < 1e-12, (P, k)


def test_grouped_equals_separate():
    """Grouping runs the same products re-batched (project page,
    'Three supporting changes', Linear layer grouping)."""
    s, W, f = small_problem(T=10, d=32, r=8, F=48, seed=4)
    a = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    b = ob.block_forward_grouped(W, f["X"], f["O"], s.D, EPS)
    for k in a:
        assert rel_err(b[k], a[k]) < 1e-13, k


def test_recompute_backward_equals_tape_backward_bitwise():
    """Checkpointing stores only the r-wide activations; the recomputed
    chunk reproduces the stored one (project page, 'Three supporting
    changes', Checkpointing without communication)."""
    s, W, f = small_problem(T=8, d=32, r=8, F=40, seed=6)
    tape = ob.block_forward(W, f["X"], f["O"], s.D, EPS, tape=True)
    saved = {k: tape[k] for k in ("q_r", "k_r", "v_r", "o_r", "g_r", "u_r",
                                  "d_r", "rms1", "rms2")}
    g1 = ob.block_backward_tape(W, tape, f["X"], f["O"], f["dY"], f["dQ"],
                                f["dK"], f["dV"], s.D)
    g2 = ob.block_backward(W, f["X"], f["O"], saved, f["dY"], f["dQ"], f["dK"],
                           f["dV"], s.D, EPS)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k
    # saved set is 7r values per token plus the two row statistics
    r = W["A_q"].shape[0]
    assert sum(saved[k].shape[1] for k in saved if k.endswith("_r")) == 7 * r


def test_textbook_special_case_full_rank_layers():
    """r = d with identity down-projections: each pair is the full-rank
    layer B (and B_dn = I makes the MLP down layer the full-rank A_dn)."""
    s, W, f = small_problem(T=5, d=8, r=8, F=16, seed=8)
    I = np.eye(8)
    for n in ("A_q", "A_k", "A_v", "A_o", "A_g", "A_u"):
        W[n] = I.copy()
    W["B_dn"] = I.copy()
    fwd = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    X, O = f["X"], f["O"]
    xn = W["gamma1"] * X / np.sqrt(np.mean(X * X, axis=1, keepdims=True) + EPS)
    h = X + O @ W["B_o"].T
    hn = W["gamma2"] * h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + EPS)
    gate, up = hn @ W["B_g"].T, hn @ W["B_u"].T
    Y = h + ((gate / (1 + np.exp(-gate))) * up) @ W["A_dn"].T
    assert rel_err(fwd["Q"], xn @ W["B_q"].T) < 1e-14
    assert rel_err(fwd["Y"], Y) < 1e-14


def test_lowrank_equals_dense_product():
    s, W, f = small_problem(T=6, d=16, r=4, F=24, seed=9)
    fwd = ob.block_forward(W, f["X"], f["O"], s.D, EPS, tape=True)
    for a, b, inp, out in (("A_q", "B_q", "xn", "Q"), ("A_o", "B_o", None, None)):
        dense = W[b] @ W[a]
        if inp:
            assert rel_err(fwd[inp] @ dense.T, fwd[out]) < 1e-12
    dense_o = W["B_o"] @ W["A_o"]
    assert rel_err(f["X"] + f["O"] @ dense_o.T, fwd["h"]) < 1e-12


@pytest.mark.parametrize("k", [2, 4])
def test_tp_rank_shares_sum_to_unsharded(k):
    """Bottleneck-aware TP: k ranks with one sum per chunk reproduce the
    unsharded block, forward and backward (project page, 'Move the chunk
    boundary to the bottleneck')."""
    s, W, f = small_problem(T=6, d=16, r=4, F=24, seed=10 + k)
    ref = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    outs, parts = osh.simulate_tp_forward(W, f["X"], f["O"], k, s.D, EPS)
    for o, (Wi, S, _) in zip(outs, parts):
        for n in ("Q", "K", "V", "Y"):
            assert rel_err(o[n], ref[n][:, S]) < 1e-12
        for n in ("q_r", "o_r", "g_r", "d_r", "rms1", "rms2"):
            assert rel_err(o[n], ref[n]) < 1e-12
    # the partials of the norm chunks add up to the unscaled product
    P_sum = sum(o["P_qkv"] for o in outs)
    assert rel_err(P_sum / ref["rms1"][:, None],
                   np.concatenate([ref["q_r"], ref["k_r"], ref["v_r"]], axis=1)) < 1e-12
    assert np.allclose(sum(o["ss1"] for o in outs), np.sum(f["X"] ** 2, axis=1))
    gref = ob.block_backward(W, f["X"], f["O"], ref, f["dY"], f["dQ"], f["dK"],
                             f["dV"], s.D, EPS)
    gr, parts = osh.simulate_tp_backward(W, f["X"], f["O"], ref, f["dY"], f["dQ"],
                                         f["dK"], f["dV"], k, s.D)
    for g, (Wi, S, SF) in zip(gr, parts):
        assert rel_err(g["X"], gref["X"][:, S]) < 1e-12
        assert rel_err(g["O"], gref["O"][:, S]) < 1e-12
        assert rel_err(g["gamma1"], gref["gamma1"][S]) < 1e-12
        for n in ("A_q", "A_o", "A_g", "A_u"):
            assert rel_err(g[n], gref[n][:, S]) < 1e-12, n
        for n in ("B_q", "B_o", "B_dn"):
            assert rel_err(g[n], gref[n][S, :]) < 1e-12, n
        assert rel_err(g["B_g"], gref["B_g"][SF, :]) < 1e-12
        assert rel_err(g["A_dn"], gref["A_dn"][:, SF]) < 1e-12


def test_rmsnorm_backward_statistic_from_r_wide_tensors():
    """sum_k dhn * hn = sum_j dz_r * z_r when z_r = hn A^T and dhn = dz_r A."""
    rng = np.random.default_rng(12)
    T, d, r = 9, 32, 6
    hn = rng.standard_normal((T, d))
    A = rng.standard_normal((r, d))
    dz = rng.standard_normal((T, r))
    lhs = np.sum((dz @ A) * hn, axis=1)
    rhs = np.sum(dz * (hn @ A.T), axis=1)
    assert rel_err(rhs, lhs) < 1e-12


# --------------------------------------------- mistakes planted in the oracle
def _torch_mismatch(monkeypatch, target, replacement):
    monkeypatch.setattr(target[0], target[1], replacement)
    s, W, f = small_problem(T=6, d=16, r=4, F=24, seed=13)
    fwd = ob.block_forward(W, f["X"], f["O"], s.D, EPS)
    G = ob.block_backward(W, f["X"], f["O"], fwd, f["dY"], f["dQ"], f["dK"],
                          f["dV"], s.D, EPS)
    tf, tg = torch_block(W, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"], EPS)
    worst = max(rel_err(fwd[k], tf[k]) for k in ("Q", "K", "V", "Y"))
    worst = max([worst] + [rel_err(G[k], tg[k]) for k in ("X", "O") + W_NAMES])
    return worst


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle; the torch pin must see each."""
    real_silu_grad = ob.silu_grad
    real_rms = ob.rms
    real_rbw = ob._rmsnorm_backward
    real_h = ob._recompute_h
    cases = {
        "dsilu drops z(1-s)": ((ob, "silu_grad"),
                               lambda z: 1.0 / (1.0 + np.exp(-z))),
        "rms with the wrong epsilon": ((ob, "rms"),
                           lambda x, D, eps: np.sqrt(np.sum(x * x, axis=1) / D + 0.5)),
        "norm bwd drops the statistic": (
            (ob, "_rmsnorm_backward"),
            lambda x, g, r, dxn, D: (g[None, :] * dxn / r[:, None],
                                     real_rbw(x, g, r, dxn, D)[1])),
        "norm bwd wrong sign": (
            (ob, "_rmsnorm_backward"),
            lambda x, g, r, dxn, D: (2 * g[None, :] * dxn / r[:, None]
                                     - real_rbw(x, g, r, dxn, D)[0],
                                     real_rbw(x, g, r, dxn, D)[1])),
        "residual missing": ((ob, "_recompute_h"),
                             lambda W, X, o_r: o_r @ W["B_o"].T),
    }
    for name, (target, repl) in cases.items():
        with monkeypatch.context() as mp:
            worst = _torch_mismatch(mp, target, repl)
        assert worst > 1e-6, name
    assert ob.silu_grad is real_silu_grad and ob.rms is real_rms
    assert ob._recompute_h is real_h
    # the unmodified oracle passes the same check
    with monkeypatch.context() as mp:
        assert _torch_mismatch(mp, (ob, "silu"), ob.silu) < 1e-12


def test_primitives_agree_with_block_oracle():
    """The standalone GEMM definitions reproduce the block's own products."""
    from oracle import primitives as op
    s, W, f = small_problem(T=7, d=16, r=4, F=24, seed=14)
    t = ob.block_forward(W, f["X"], f["O"], s.D, EPS, tape=True)
    G = ob.block_backward_tape(W, t, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"], s.D)
    Q, K, V = op.grouped_gemm("NT", [(t["q_r"], W["B_q"]), (t["k_r"], W["B_k"]),
                                     (t["v_r"], W["B_v"])])
    assert rel_err(Q, t["Q"]) < 1e-14 and rel_err(V, t["V"]) < 1e-14
    (m,) = op.grouped_gemm("NT", [(t["g_r"], W["B_g"]), (t["u_r"], W["B_u"])], "swiglu")
    assert rel_err(m, t["m"]) < 1e-14
    (h,) = op.grouped_gemm("NT", [(t["o_r"], W["B_o"])], "residual", f["X"])
    assert rel_err(h, t["h"]) < 1e-14
    (dBdn,) = op.grouped_gemm("TN", [(f["dY"], t["d_r"])])
    assert rel_err(dBdn, G["B_dn"]) < 1e-14
    (xn_like,) = op.grouped_gemm("NN", [(f["X"], np.eye(16))], "row_scale", t["rms1"])
    assert rel_err(W["gamma1"] * xn_like, t["xn"]) < 1e-14
