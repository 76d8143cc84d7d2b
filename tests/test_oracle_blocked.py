"""Pins of the oracle's row-blocked driver, ``oracle.run_fwd_bwd``.

Every GPU parity test, the smoke check and the bench's cpu_baseline go
through this driver, so it is pinned here on its own: with a token count
that is not a multiple of the row block (13 tokens in blocks of 4: three
whole blocks and a one-row tail), in the plain, 2-panel and rank-share
modes, every row-local output, per-panel sum, partial and accumulated weight
or gamma gradient is compared with

  * one unblocked call of the pinned block functions (``block_forward``,
    ``block_forward_online``, ``share_forward``, ``block_backward`` and, for
    the rank share, ``share_backward``), assembled into the grouped layouts
    here, and
  * torch's float64 ``rms_norm``/``linear``/``silu`` with autograd (zero-padded
    to the divisor D for the rank share).

The weight gradients are sums over every token (project page, "Three
supporting changes": the factors see all rows), so a driver that overwrote
instead of adding a block's part, paired the rank share's forward with a
backward of the wrong divisor, or mixed up the panels of the per-panel sums
fails here (a driver that returned them untransposed fails the shape check);
each of those mistakes is planted below and must be caught.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import block as ob
from oracle import blocked as obk
from oracle import share as osh
from tests.oracle_helpers import W_NAMES, rel_err, small_problem, torch_block

EPS = 1e-5
T_ROWS, ROW_BLOCK = 13, 4

MODES = {
    "plain": dict(shape=dict(T=T_ROWS, d=16, r=4, F=24, seed=21), P=1, partials=False),
    "panels": dict(shape=dict(T=T_ROWS, d=16, r=4, F=24, seed=22), P=2, partials=False),
    "partials": dict(shape=dict(T=T_ROWS, d=12, r=6, F=20, D=48, seed=23), P=1, partials=True),
}
WGRAD_KEYS = ("dgamma1", "dgamma2", "dA_qkv", "dB_q", "dB_k", "dB_v", "dA_o", "dB_o",
              "dA_gu", "dB_g", "dB_u", "dA_dn", "dB_dn")


def _grad_layout(G):
    """Gradients under the driver's names and grouped layouts."""
    return dict(
        dX=G["X"], dO=G["O"], dgamma1=G["gamma1"], dgamma2=G["gamma2"],
        dA_qkv=np.concatenate([G["A_q"], G["A_k"], G["A_v"]], axis=0),
        dB_q=G["B_q"], dB_k=G["B_k"], dB_v=G["B_v"], dA_o=G["A_o"], dB_o=G["B_o"],
        dA_gu=np.concatenate([G["A_g"], G["A_u"]], axis=0),
        dB_g=G["B_g"], dB_u=G["B_u"], dA_dn=G["A_dn"], dB_dn=G["B_dn"])


def _unblocked(mode):
    """Expected outputs from one call of the pinned functions on all rows."""
    cfg = MODES[mode]
    s, W, f = small_problem(**cfg["shape"])
    X, O = f["X"], f["O"]
    ups = (f["dY"], f["dQ"], f["dK"], f["dV"])
    if cfg["partials"]:
        fwd = osh.share_forward(W, X, O, s.D, EPS)
        G = osh.share_backward(W, X, O, fwd, *ups, s.D)
    elif cfg["P"] > 1:
        fwd = ob.block_forward_online(W, X, O, s.D, EPS, cfg["P"])
        G = ob.block_backward(W, X, O, fwd, *ups, s.D, EPS)
    else:
        fwd = ob.block_forward(W, X, O, s.D, EPS)
        G = ob.block_backward(W, X, O, fwd, *ups, s.D, EPS)
    exp = dict(Q=fwd["Q"], K=fwd["K"], V=fwd["V"], Y=fwd["Y"], o_r=fwd["o_r"],
               d_r=fwd["d_r"], rms1=fwd["rms1"], rms2=fwd["rms2"],
               qkv_r=np.concatenate([fwd["q_r"], fwd["k_r"], fwd["v_r"]], axis=1),
               gu_r=np.concatenate([fwd["g_r"], fwd["u_r"]], axis=1))
    if cfg["P"] > 1:
        exp["ss_panels1"], exp["ss_panels2"] = fwd["ss_panels1"], fwd["ss_panels2"]
    if cfg["partials"]:
        for k in ("P_qkv", "ss1", "P_gu", "ss2"):
            exp[k] = fwd[k]
    exp.update(_grad_layout(G))
    return s, W, f, exp


def _run_driver(mode, f, s, **kw):
    cfg = MODES[mode]
    return oracle.run_fwd_bwd(f, D=s.D, eps=EPS, n_panels=cfg["P"], partials=cfg["partials"],
                              row_block=ROW_BLOCK, **kw)


def _worst(got, exp):
    bad = {}
    for k, v in exp.items():
        assert k in got, k
        assert np.shape(got[k]) == np.shape(v), (k, np.shape(got[k]), np.shape(v))
        bad[k] = rel_err(got[k], v)
    assert set(got) == set(exp), set(got) ^ set(exp)
    return bad


@pytest.mark.parametrize("mode", list(MODES))
def test_row_blocked_driver_matches_unblocked_functions(mode):
    s, W, f, exp = _unblocked(mode)
    assert s.T % ROW_BLOCK != 0
    got = _run_driver(mode, f, s)
    errs = _worst(got, exp)
    # Blocking only splits the sums over tokens (the weight gradients) into
    # partial sums; every other value is computed row by row.
    for k, e in errs.items():
        assert e < 1e-13, (k, e)


@pytest.mark.parametrize("mode", list(MODES))
def test_row_blocked_driver_matches_torch_autograd(mode):
    s, W, f, _ = _unblocked(mode)
    got = _run_driver(mode, f, s)
    tf, tg = torch_block(W, f["X"], f["O"], f["dY"], f["dQ"], f["dK"], f["dV"], EPS,
                         D=s.D if s.D != s.d else None)
    for k in ("Q", "K", "V", "Y"):
        assert rel_err(got[k], tf[k]) < 1e-12, k
    want = _grad_layout(tg)
    for k in ("dX", "dO") + WGRAD_KEYS:
        assert rel_err(got[k], want[k]) < 1e-12, k


@pytest.mark.parametrize("mode", list(MODES))
def test_row_blocked_driver_sampled_rows_and_callback(mode):
    """The ``rows`` and ``on_rows`` paths give the same row-local values."""
    s, W, f, exp = _unblocked(mode)
    rows = np.array([12, 0, 5, 6, 7, 11])
    got = _run_driver(mode, f, s, rows=rows)
    for k in WGRAD_KEYS:
        assert k not in got
    for k, v in got.items():
        ref = exp[k][:, rows] if k.startswith("ss_panels") else exp[k][rows]
        assert rel_err(v, ref) < 1e-13, k
    seen = {}

    def on_rows(sel, loc):
        for k, v in loc.items():
            seen.setdefault(k, []).append((np.array(sel), v))

    out = _run_driver(mode, f, s, on_rows=on_rows)
    assert set(out) == set(WGRAD_KEYS)
    for k, parts in seen.items():
        assert sum(len(sel) for sel, _ in parts) == s.T
        for sel, v in parts:
            ref = exp[k][:, sel].T if k.startswith("ss_panels") else exp[k][sel]
            assert rel_err(v, ref) < 1e-13, k


# --------------------------------------------- mistakes planted in the driver
def test_driver_pins_catch_planted_mistakes(monkeypatch):
    def overwrite(acc, grads):  # keeps only the last row block's part
        acc.update(grads)

    real_bwd = obk.block_backward

    def wrong_divisor(W, X, O, saved, dY, dQ, dK, dV, D, eps):  # the rank's width, not D
        return real_bwd(W, X, O, saved, dY, dQ, dK, dV, X.shape[1], eps)

    real_online = obk.block_forward_online

    def panels_reversed(*a, **k):  # per-panel sums indexed P - 1 - p
        out = real_online(*a, **k)
        out["ss_panels1"] = np.ascontiguousarray(out["ss_panels1"][::-1])
        return out

    cases = {
        "overwrite instead of accumulate": ("plain", (obk, "_accumulate", overwrite)),
        "rank share with the wrong backward": ("partials", (obk, "block_backward", wrong_divisor)),
        "panel sums in the wrong order": ("panels", (obk, "block_forward_online", panels_reversed)),
    }
    for name, (mode, (mod, attr, repl)) in cases.items():
        s, W, f, exp = _unblocked(mode)
        with monkeypatch.context() as mp:
            mp.setattr(mod, attr, repl)
            got = _run_driver(mode, f, s)
        errs = _worst(got, exp)
        assert max(errs.values()) > 1e-3, name
    # the unmodified driver passes the same comparison
    s, W, f, exp = _unblocked("plain")
    assert max(_worst(_run_driver("plain", f, s), exp).values()) < 1e-13
