"""The whole decoder block through the C ABI: the block's pre-attention
stage, causal RoPE attention, the post-attention stage, and back
(lr_block_fwd/bwd with LR_STAGE_PRE_ATTN / LR_STAGE_POST_ATTN around
lr_attention_fwd/bwd), against the same composition of the fp64 oracles:
the block oracle (oracle.run_fwd_bwd) with O and dQ, dK, dV supplied by
the attention oracle (oracle/attention.py)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from oracle import attention as oa
from tests.gpu_helpers import BF16_TOL, ErrAcc, gpu_or_skip, say

pytestmark = pytest.mark.gpu

DH = 128


def _oracle_block_with_attention(inp, s, seq_len, heads, base):
    """Oracle composition: Q, K, V from the block, O from attention, dO from
    the block's post-attention backward, dQ, dK, dV from attention's
    backward, then the block's full backward."""
    zeros = np.zeros_like(inp["X"], dtype=np.float64)
    kw = dict(D=s.D, eps=s.eps, n_panels=s.P, partials=False)
    first = oracle.run_fwd_bwd({**inp, "O": zeros, "dQ": zeros, "dK": zeros, "dV": zeros},
                               backward=False, **kw)
    Q, K, V = first["Q"], first["K"], first["V"]
    O, lse = oa.attention_forward(Q, K, V, seq_len, heads, heads, DH, base)
    second = oracle.run_fwd_bwd({**inp, "O": O, "dQ": zeros, "dK": zeros, "dV": zeros},
                                weight_grads=False, **kw)
    dQ, dK, dV = oa.attention_backward(Q, K, V, second["dO"], seq_len, heads, heads, DH, base)
    full = oracle.run_fwd_bwd({**inp, "O": O, "dQ": dQ, "dK": dK, "dV": dV}, **kw)
    full["O"], full["lse"] = O, lse
    full["dQ_attn"], full["dK_attn"], full["dV_attn"] = dQ, dK, dV
    return full


@pytest.mark.parametrize("n_seq,seq_len", [(2, 256), (3, 200)])
def test_block_with_attention_matches_oracle(n_seq, seq_len):
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    from gemm_online_rmsnorm_amd.runner import BlockRun

    heads, base = 2, 10000.0
    d = heads * DH
    s = synth.BlockShape("block+attention", T=n_seq * seq_len, d=d, r=64, F=688, D=d, P=1,
                         seed=21)
    say(f"[block+attention] T={s.T} seq_len={seq_len} d={d} heads={heads}")
    inp = synth.make_inputs(s)
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials, inp)
    ashape = lr.attn_shape(s.T, seq_len, heads, heads, DH, base)
    lse = torch.empty(heads, s.T, dtype=torch.float32, device="cuda")

    run.fwd(stage=lr.LR_STAGE_PRE_ATTN)
    Q, K, V = run.out["Q"], run.out["K"], run.out["V"]
    lr.attention_fwd(ashape, Q, K, V, run.O, lse)
    run.fwd(stage=lr.LR_STAGE_POST_ATTN)
    run.bwd(stage=lr.LR_STAGE_POST_ATTN)
    lr.attention_bwd(ashape, Q, K, V, run.O, run.dO, lse, run.dQ, run.dK, run.dV)
    run.bwd(stage=lr.LR_STAGE_PRE_ATTN)
    got = run.results()
    got["O"] = run.O.float().cpu().numpy().astype(np.float64)
    got["lse"] = lse.cpu().numpy().astype(np.float64)

    ref = _oracle_block_with_attention(inp, s, seq_len, heads, base)
    acc = ErrAcc()
    for name in ("Q", "K", "V", "O", "lse", "Y", "dO", "dX", "qkv_r", "o_r", "gu_r", "d_r",
                 "rms1", "rms2", "dgamma1", "dgamma2", "dA_qkv", "dB_q", "dB_k", "dB_v",
                 "dA_o", "dB_o", "dA_gu", "dB_g", "dB_u", "dA_dn", "dB_dn"):
        acc.add(name, got[name], ref[name])
    acc.check(BF16_TOL, f"block+attention T={s.T}")
