"""fp64 causal self-attention with rotary position embedding, multi-head or
grouped-query (TEST INFRASTRUCTURE ONLY, like the rest of this package).

The BOOST pages leave the attention core of the LLaMA-style block outside
the method (their block diagram runs the factorised linear layers around
it, their related-work list cites FlashAttention and grouped-query
attention, and the project page's scope section says the design is argued,
not tested, for grouped-query attention). This module therefore writes out
the textbook definitions the LLaMA-2 family uses, which the pages do not
restate:

* rotary embedding (RoPE) in the half-split form: for head dimension dh and
  i < dh / 2, the pair (x_i, x_{i + dh/2}) of a token at position p is
  rotated by the angle p * base^(-2i/dh);
* per sequence and head, S = q k^T / sqrt(dh) with q, k rotated; keys after
  the query's own position are masked (causal); P = softmax over keys;
  O = P v. Query head h reads key/value head h // (H / H_kv) (grouped-query
  attention; H_kv = H is multi-head attention);
* LSE = log(sum_j exp S_ij) per query row (natural log), the statistic a
  fused backward needs;
* the backward of the above: dV = P^T dO, dP = dO v^T,
  dS = P * (dP - rowsum(dO * O)), dq = dS k / sqrt(dh),
  dk = dS^T q / sqrt(dh), then the transposed rotation on dq and dk; the
  query heads of a group add their dk and dv.

Layout (the block's): Q [T, H * dh], K and V [T, H_kv * dh], token-major,
head h in columns [h dh, (h + 1) dh); the T tokens are n_seq sequences of
seq_len consecutive tokens, positions 0 .. seq_len - 1 within each.

Parity status: pinned by tests/test_oracle_attention.py (closed forms of
the rotation and of uniform attention, the adjoint identity of the
rotation, torch's scaled_dot_product_attention and autograd, finite
differences).
"""
from __future__ import annotations

import numpy as np


def rope_angles(seq_len: int, dh: int, base: float) -> np.ndarray:
    """[seq_len, dh/2] angles p * base^(-2i/dh)."""
    i = np.arange(dh // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / dh)
    return np.arange(seq_len, dtype=np.float64)[:, None] * inv[None, :]


def rope(x: np.ndarray, base: float, inverse: bool = False) -> np.ndarray:
    """Rotate x [seq_len, heads, dh] by position; inverse=True applies the
    transposed (inverse) rotation, the backward of the forward one."""
    x = np.asarray(x, dtype=np.float64)
    S, _, dh = x.shape
    a = rope_angles(S, dh, base)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    if inverse:
        s = -s
    x1, x2 = x[..., : dh // 2], x[..., dh // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _split(X, seq_len, heads, dh):
    X = np.asarray(X, dtype=np.float64)
    return X.reshape(X.shape[0] // seq_len, seq_len, heads, dh)


def attention_forward(Q, K, V, seq_len: int, n_heads: int, n_kv_heads: int, dh: int,
                      base: float):
    """O [T, H dh] and LSE [H, T] of causal RoPE attention."""
    q = _split(Q, seq_len, n_heads, dh)
    k = _split(K, seq_len, n_kv_heads, dh)
    v = _split(V, seq_len, n_kv_heads, dh)
    nseq = q.shape[0]
    grp = n_heads // n_kv_heads
    O = np.zeros_like(q)
    lse = np.zeros((n_heads, nseq, seq_len))
    mask = np.triu(np.ones((seq_len, seq_len), dtype=bool), 1)
    for b in range(nseq):
        qr = rope(q[b], base)
        kr = rope(k[b], base)
        for h in range(n_heads):
            hk = h // grp
            S = qr[:, h, :] @ kr[:, hk, :].T / np.sqrt(dh)
            S[mask] = -np.inf
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            z = E.sum(axis=1, keepdims=True)
            O[b, :, h, :] = (E / z) @ v[b, :, hk, :]
            lse[h, b, :] = (m + np.log(z))[:, 0]
    return O.reshape(nseq * seq_len, n_heads * dh), lse.reshape(n_heads, nseq * seq_len)


def attention_backward(Q, K, V, dO, seq_len: int, n_heads: int, n_kv_heads: int, dh: int,
                       base: float):
    """dQ [T, H dh], dK and dV [T, H_kv dh] of attention_forward."""
    q = _split(Q, seq_len, n_heads, dh)
    k = _split(K, seq_len, n_kv_heads, dh)
    v = _split(V, seq_len, n_kv_heads, dh)
    do = _split(dO, seq_len, n_heads, dh)
    nseq = q.shape[0]
    grp = n_heads // n_kv_heads
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mask = np.triu(np.ones((seq_len, seq_len), dtype=bool), 1)
    for b in range(nseq):
        qr = rope(q[b], base)
        kr = rope(k[b], base)
        dqr = np.zeros_like(qr)
        dkr = np.zeros_like(kr)
        for h in range(n_heads):
            hk = h // grp
            S = qr[:, h, :] @ kr[:, hk, :].T / np.sqrt(dh)
            S[mask] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            o = P @ v[b, :, hk, :]
            dv[b, :, hk, :] += P.T @ do[b, :, h, :]
            dP = do[b, :, h, :] @ v[b, :, hk, :].T
            dS = P * (dP - (do[b, :, h, :] * o).sum(axis=1, keepdims=True))
            dqr[:, h, :] = dS @ kr[:, hk, :] / np.sqrt(dh)
            dkr[:, hk, :] += dS.T @ qr[:, h, :] / np.sqrt(dh)
        dq[b] = rope(dqr, base, inverse=True)
        dk[b] = rope(dkr, base, inverse=True)
    T = nseq * seq_len
    return (dq.reshape(T, n_heads * dh), dk.reshape(T, n_kv_heads * dh),
            dv.reshape(T, n_kv_heads * dh))
