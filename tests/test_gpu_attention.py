"""Parity of the causal RoPE attention entry points (lr_attention_fwd,
lr_attention_bwd) with the fp64 oracle (oracle/attention.py): whole outputs
on small ragged shapes (multi-head, grouped-query, multi-query, one-token
sequences), and at the LLaMA-2-7B shape (4 x 4096 tokens, 32 heads of 128)
computed in the launch configuration the benchmark times: every head of one
sequence and one head group of each other sequence."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import attention as oa
from tests.gpu_helpers import BF16_TOL, ErrAcc, gpu_or_skip, say

pytestmark = pytest.mark.gpu

DH = 128


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run(torch, s, inp):
    """Forward and backward through the C ABI; returns host fp64 arrays."""
    import gemm_online_rmsnorm_amd as lr
    shape = lr.attn_shape(s.T, s.seq_len, s.H, s.Hkv, DH, s.base)
    Q, K, V, dO = (_dev(torch, inp[n]) for n in ("Q", "K", "V", "dO"))
    O = torch.empty_like(Q)
    lse = torch.empty(s.H, s.T, dtype=torch.float32, device="cuda")
    lr.attention_fwd(shape, Q, K, V, O, lse)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    lr.attention_bwd(shape, Q, K, V, O, dO, lse, dQ, dK, dV)
    torch.cuda.synchronize()
    return {"O": _host(O), "lse": lse.cpu().numpy().astype(np.float64), "dQ": _host(dQ),
            "dK": _host(dK), "dV": _host(dV)}


SMALL = [
    synth.AttnShape("mha ragged", T=400, seq_len=200, H=2, Hkv=2, seed=1),
    synth.AttnShape("gqa", T=640, seq_len=320, H=4, Hkv=2, seed=2),
    synth.AttnShape("mqa odd heads", T=192, seq_len=192, H=3, Hkv=1, seed=3),
    synth.AttnShape("one-token sequences", T=5, seq_len=1, H=2, Hkv=1, seed=4),
    synth.AttnShape("short sequences", T=111, seq_len=37, H=2, Hkv=2, seed=5),
    synth.AttnShape("long ragged", T=1100, seq_len=1100, H=2, Hkv=1, seed=6),
    synth.AttnShape("rope base 500000", T=256, seq_len=256, H=2, Hkv=2, base=500000.0, seed=7),
    # tile edges: 64-row K/V and query tiles, 128-row query and key blocks
    synth.AttnShape("seq 64", T=192, seq_len=64, H=2, Hkv=1, seed=8),
    synth.AttnShape("seq 127", T=254, seq_len=127, H=2, Hkv=2, seed=9),
    synth.AttnShape("seq 128", T=256, seq_len=128, H=1, Hkv=1, seed=10),
    synth.AttnShape("seq 129", T=258, seq_len=129, H=8, Hkv=1, seed=11),
    # long sequence: positions up to 8191 (large rotation angles), 128 key tiles
    synth.AttnShape("seq 8192", T=8192, seq_len=8192, H=2, Hkv=1, seed=12),
]


@pytest.mark.parametrize("s", SMALL, ids=[s.name for s in SMALL])
def test_attention_matches_oracle(s):
    torch = gpu_or_skip()
    say(f"[attention] {s.name}: T={s.T} seq_len={s.seq_len} H={s.H} Hkv={s.Hkv}")
    inp = synth.make_attn_inputs(s)
    got = _run(torch, s, inp)
    args = (s.seq_len, s.H, s.Hkv, DH, s.base)
    O, lse = oa.attention_forward(inp["Q"], inp["K"], inp["V"], *args)
    dQ, dK, dV = oa.attention_backward(inp["Q"], inp["K"], inp["V"], inp["dO"], *args)
    acc = ErrAcc()
    for name, ref in (("O", O), ("lse", lse), ("dQ", dQ), ("dK", dK), ("dV", dV)):
        acc.add(name, got[name], ref)
    acc.check(BF16_TOL, s.name)


def test_one_token_sequences_return_v():
    """seq_len = 1: each token attends only to itself, so O = V of its
    key/value head and LSE = q.k / sqrt(128) of the rotation-free
    position 0."""
    torch = gpu_or_skip()
    s = synth.AttnShape("one token", T=7, seq_len=1, H=4, Hkv=2, seed=9)
    inp = synth.make_attn_inputs(s)
    got = _run(torch, s, inp)
    grp = s.H // s.Hkv
    for h in range(s.H):
        hk = h // grp
        v = inp["V"][:, hk * DH:(hk + 1) * DH]
        assert np.allclose(got["O"][:, h * DH:(h + 1) * DH], v, rtol=1e-2, atol=1e-2)
        q = inp["Q"][:, h * DH:(h + 1) * DH].astype(np.float64)
        k = inp["K"][:, hk * DH:(hk + 1) * DH].astype(np.float64)
        assert np.allclose(got["lse"][h], np.sum(q * k, axis=1) / np.sqrt(DH), rtol=1e-2,
                           atol=2e-2)


def _slice(a, b, S, h0, nh):
    return a[b * S:(b + 1) * S, h0 * DH:(h0 + nh) * DH]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("s", [synth.ATTN_7B, synth.ATTN_7B_GQA], ids=["mha", "gqa"])
def test_full_size_every_head_of_one_sequence_and_a_group_of_each_other(s):
    """Full LLaMA-2-7B shape in the launch configuration the benchmark
    times. The oracle recomputes every query and key/value head of the first
    sequence, and one key/value head with its query heads of every other
    sequence (a different head in each); the outputs of a (sequence, head
    group) depend on nothing else. Every other output is checked finite."""
    torch = gpu_or_skip()
    say(f"[attention full] {s.name}")
    inp = synth.make_attn_inputs(s)
    got = _run(torch, s, inp)
    for name in ("O", "lse", "dQ", "dK", "dV"):
        assert np.all(np.isfinite(got[name])), name
    grp = s.H // s.Hkv
    S = s.seq_len
    # (sequence, first kv head, kv heads): all of sequence 0, then one group
    # of each other sequence
    parts = [(0, 0, s.Hkv)] + [(b, (5 * b + 1) % s.Hkv, 1) for b in range(1, s.n_seq)]
    for b, hk, nk in parts:
        q = _slice(inp["Q"], b, S, hk * grp, nk * grp)
        k = _slice(inp["K"], b, S, hk, nk)
        v = _slice(inp["V"], b, S, hk, nk)
        do = _slice(inp["dO"], b, S, hk * grp, nk * grp)
        args = (S, nk * grp, nk, DH, s.base)
        O, lse = oa.attention_forward(q, k, v, *args)
        dQ, dK, dV = oa.attention_backward(q, k, v, do, *args)
        acc = ErrAcc()
        acc.add("O", _slice(got["O"], b, S, hk * grp, nk * grp), O)
        acc.add("lse", got["lse"][hk * grp:(hk + nk) * grp, b * S:(b + 1) * S], lse)
        acc.add("dQ", _slice(got["dQ"], b, S, hk * grp, nk * grp), dQ)
        acc.add("dK", _slice(got["dK"], b, S, hk, nk), dK)
        acc.add("dV", _slice(got["dV"], b, S, hk, nk), dV)
        acc.check(BF16_TOL, f"{s.name} sequence {b} kv heads {hk}..{hk + nk - 1}")
