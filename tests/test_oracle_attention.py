"""Pins of the oracle's causal RoPE attention (oracle/attention.py) against
closed forms, torch's attention routine and autograd, and finite
differences (CPU only)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention as oa

BASE = 10000.0


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_rope_rotates_each_pair_by_position_times_frequency():
    S, dh = 7, 8
    x = np.zeros((S, 1, dh))
    x[:, 0, 1] = 1.0  # pair i = 1: frequency base^(-2/dh)
    y = oa.rope(x, BASE)
    ang = np.arange(S) * BASE ** (-2.0 / dh)
    assert np.allclose(y[:, 0, 1], np.cos(ang))
    assert np.allclose(y[:, 0, 1 + dh // 2], np.sin(ang))
    others = np.delete(np.arange(dh), [1, 1 + dh // 2])
    assert np.allclose(y[:, 0, others], 0.0)
    # position 0 is the identity
    z = _rand(np.random.default_rng(0), 1, 3, dh)
    assert np.allclose(oa.rope(z, BASE), z)


def test_rope_inverse_is_adjoint_and_inverse():
    rng = np.random.default_rng(1)
    x, y = _rand(rng, 9, 2, 16), _rand(rng, 9, 2, 16)
    assert np.isclose(np.sum(oa.rope(x, BASE) * y), np.sum(x * oa.rope(y, BASE, inverse=True)))
    assert np.allclose(oa.rope(oa.rope(x, BASE), BASE, inverse=True), x)
    # scores depend on relative position only
    q, k = _rand(rng, 1, 1, 16), _rand(rng, 1, 1, 16)
    qs = oa.rope(np.repeat(q, 9, 0), BASE)
    ks = oa.rope(np.repeat(k, 9, 0), BASE)
    assert np.isclose(qs[5, 0] @ ks[3, 0], qs[4, 0] @ ks[2, 0])


def test_uniform_scores_average_the_causal_prefix():
    """Q = 0: every score is 0, so row i averages the values of positions
    0 .. i of its sequence and LSE = log(i + 1)."""
    rng = np.random.default_rng(2)
    S, H, dh, nseq = 6, 2, 8, 3
    Q = np.zeros((nseq * S, H * dh))
    K = _rand(rng, nseq * S, H * dh)
    V = _rand(rng, nseq * S, H * dh)
    O, lse = oa.attention_forward(Q, K, V, S, H, H, dh, BASE)
    v = V.reshape(nseq, S, H * dh)
    want = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None]
    assert np.allclose(O, want.reshape(nseq * S, H * dh))
    assert np.allclose(lse, np.tile(np.log(np.arange(1, S + 1)), nseq)[None, :].repeat(H, 0))


def _torch_ref(Q, K, V, dO, S, H, Hkv, dh):
    """torch's causal attention on the oracle-rotated q, k; returns O, dq_rot,
    dk_rot, dv (gradients of sum(O * dO) by autograd)."""
    nseq = Q.shape[0] // S
    qs, ks, vs = [], [], []
    for b in range(nseq):
        qs.append(oa.rope(Q[b * S:(b + 1) * S].reshape(S, H, dh), BASE))
        ks.append(oa.rope(K[b * S:(b + 1) * S].reshape(S, Hkv, dh), BASE))
        vs.append(V[b * S:(b + 1) * S].reshape(S, Hkv, dh))
    q = torch.tensor(np.stack(qs).transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
    k = torch.tensor(np.stack(ks).transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
    v = torch.tensor(np.stack(vs).transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
    rep = H // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(rep, dim=1), v.repeat_interleave(rep, dim=1), is_causal=True)
    g = torch.tensor(dO.reshape(nseq, S, H, dh).transpose(0, 2, 1, 3))
    (o * g).sum().backward()

    def back(t, heads):  # [nseq, heads, S, dh] -> [nseq, S, heads, dh]
        return t.detach().numpy().transpose(0, 2, 1, 3)
    return back(o, H), back(q.grad, H), back(k.grad, Hkv), back(v.grad, Hkv)


@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_forward_and_backward_match_torch(H, Hkv):
    rng = np.random.default_rng(3 + H + Hkv)
    S, dh, nseq = 11, 8, 2
    T = nseq * S
    Q, K, V = _rand(rng, T, H * dh), _rand(rng, T, Hkv * dh), _rand(rng, T, Hkv * dh)
    dO = _rand(rng, T, H * dh)
    O, _ = oa.attention_forward(Q, K, V, S, H, Hkv, dh, BASE)
    dQ, dK, dV = oa.attention_backward(Q, K, V, dO, S, H, Hkv, dh, BASE)
    o_t, dqr, dkr, dv_t = _torch_ref(Q, K, V, dO, S, H, Hkv, dh)
    assert np.allclose(O.reshape(nseq, S, H, dh), o_t, atol=1e-12)
    assert np.allclose(dV.reshape(nseq, S, Hkv, dh), dv_t, atol=1e-12)
    for b in range(nseq):
        want_q = oa.rope(dqr[b], BASE, inverse=True)
        want_k = oa.rope(dkr[b], BASE, inverse=True)
        assert np.allclose(dQ[b * S:(b + 1) * S].reshape(S, H, dh), want_q, atol=1e-12)
        assert np.allclose(dK[b * S:(b + 1) * S].reshape(S, Hkv, dh), want_k, atol=1e-12)


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(7)
    S, H, Hkv, dh, nseq = 5, 2, 1, 4, 2
    T = nseq * S
    Q, K, V = _rand(rng, T, H * dh), _rand(rng, T, Hkv * dh), _rand(rng, T, Hkv * dh)
    G = _rand(rng, T, H * dh)

    def loss(Q, K, V):
        return np.sum(oa.attention_forward(Q, K, V, S, H, Hkv, dh, BASE)[0] * G)

    grads = oa.attention_backward(Q, K, V, G, S, H, Hkv, dh, BASE)
    eps = 1e-6
    for which, X in enumerate((Q, K, V)):
        for idx in [(0, 0), (3, 1), (T - 1, X.shape[1] - 1), (S, 2)]:
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            args_p[which], args_m[which] = Xp, Xm
            num = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(num - grads[which][idx]) < 1e-6 * max(1.0, abs(num))


def test_pins_catch_a_planted_mistake(monkeypatch):
    """A sign slip in the rotation (a plausible mistake) fails the closed-form
    pin."""
    orig = oa.rope

    def bad(x, base, inverse=False):
        return orig(x, base, inverse=not inverse)

    monkeypatch.setattr(oa, "rope", bad)
    with pytest.raises(AssertionError):
        test_rope_rotates_each_pair_by_position_times_frequency()
