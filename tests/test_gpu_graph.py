"""The entry points under HIP stream capture: a block step (lr_block_fwd +
lr_block_bwd), attention forward + backward, and the whole decoder block
(block stages around attention) are captured once into a graph
(torch.cuda.CUDAGraph, i.e. hipStreamBeginCapture / hipGraphLaunch) and
replayed several times. Before every replay the outputs are filled with NaN
by eager work on the same stream, and other eager library calls run between
the replays; each replay must reproduce the eager outputs bit for bit (the
kernels are deterministic: fixed grids, fixed reduction orders, no atomics).
The eager outputs of the block and of attention are checked against the
fp64 oracle in the same test, so a replay that matches them is within the
parity bar too."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from oracle import attention as oa
from tests.gpu_helpers import BF16_TOL, ErrAcc, gpu_or_skip, say

pytestmark = pytest.mark.gpu

DH = 128
REPLAYS = 3


def _fill_nan(ts):
    for t in ts:
        t.fill_(float("nan"))


def _same_bits(torch, got, want, label):
    for i, (g, w) in enumerate(zip(got, want)):
        assert g.shape == w.shape
        gb = g.view(torch.int16) if g.dtype == torch.bfloat16 else g.view(torch.int32)
        wb = w.view(torch.int16) if w.dtype == torch.bfloat16 else w.view(torch.int32)
        ndiff = int((gb != wb).sum().item())
        assert ndiff == 0, f"{label}: output {i} differs from the eager run in {ndiff} elements"


def _capture(torch, fn):
    """Capture fn() into a graph on a side stream (torch's capture protocol:
    one eager call on the side stream first)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(torch, g, outs, want, label, between):
    for i in range(REPLAYS):
        _fill_nan(outs)
        g.replay()
        torch.cuda.synchronize()
        _same_bits(torch, outs, want, f"{label} replay {i}")
        between()          # eager library work between replays
        torch.cuda.synchronize()


def _block_outputs(run):
    outs = list(run.out.values()) + list(run.saved.values()) + [run.dX, run.dO]
    outs += list(run.grads.values())
    if run.part is not None:
        outs += list(run.part.values())
    return outs


def test_block_step_graph_replay():
    torch = gpu_or_skip()
    from gemm_online_rmsnorm_amd.runner import BlockRun

    s = synth.BlockShape("graph block", T=640, d=512, r=128, F=1376, D=512, P=1, seed=31)
    say(f"[graph] block step T={s.T} d={s.d} r={s.r} F={s.F}")
    inp = synth.make_inputs(s)
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials, inp)
    other = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials,
                     synth.make_inputs(s, seed=32))

    run.step()
    got = run.results()
    ref = oracle.run_fwd_bwd(inp, D=s.D, eps=s.eps, n_panels=s.P, partials=False)
    acc = ErrAcc()
    for name in ("Q", "K", "V", "Y", "dX", "dO", "qkv_r", "o_r", "gu_r", "d_r", "rms1",
                 "rms2", "dgamma1", "dA_qkv", "dB_q", "dB_o", "dA_gu", "dB_g", "dB_u",
                 "dA_dn", "dB_dn"):
        acc.add(name, got[name], ref[name])
    acc.check(BF16_TOL, "eager block step")

    outs = _block_outputs(run)
    want = [t.clone() for t in outs]
    g = _capture(torch, run.step)
    _replay_and_check(torch, g, outs, want, "block step", other.step)


def test_attention_graph_replay():
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr

    s = synth.AttnShape("graph attention", T=600, seq_len=300, H=4, Hkv=2, seed=33)
    say(f"[graph] attention T={s.T} seq_len={s.seq_len} H={s.H} Hkv={s.Hkv}")
    inp = synth.make_attn_inputs(s)
    shape = lr.attn_shape(s.T, s.seq_len, s.H, s.Hkv, DH, s.base)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(
            torch.bfloat16)

    Q, K, V, dO = (dev(inp[n]) for n in ("Q", "K", "V", "dO"))
    O = torch.empty_like(Q)
    lse = torch.empty(s.H, s.T, dtype=torch.float32, device="cuda")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ws_f = torch.empty(lr.attention_workspace_bytes(shape, False), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(lr.attention_workspace_bytes(shape, True), dtype=torch.uint8,
                       device="cuda")

    def step():
        lr.attention_fwd(shape, Q, K, V, O, lse, ws_f)
        lr.attention_bwd(shape, Q, K, V, O, dO, lse, dQ, dK, dV, ws_b)

    # Eager work between replays: the same entry points on other buffers.
    Q2, K2, V2 = Q.flip(0).contiguous(), K.flip(0).contiguous(), V.flip(0).contiguous()
    O2, lse2 = torch.empty_like(Q), torch.empty_like(lse)
    dQ2, dK2, dV2 = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)

    def between():
        lr.attention_fwd(shape, Q2, K2, V2, O2, lse2)
        lr.attention_bwd(shape, Q2, K2, V2, O2, dO, lse2, dQ2, dK2, dV2)

    step()
    torch.cuda.synchronize()
    args = (s.seq_len, s.H, s.Hkv, DH, s.base)
    rO, rlse = oa.attention_forward(inp["Q"], inp["K"], inp["V"], *args)
    rdQ, rdK, rdV = oa.attention_backward(inp["Q"], inp["K"], inp["V"], inp["dO"], *args)
    acc = ErrAcc()
    for name, t, r in (("O", O, rO), ("lse", lse, rlse), ("dQ", dQ, rdQ), ("dK", dK, rdK),
                       ("dV", dV, rdV)):
        acc.add(name, t.float().cpu().numpy(), r)
    acc.check(BF16_TOL, "eager attention")

    outs = [O, lse, dQ, dK, dV]
    want = [t.clone() for t in outs]
    g = _capture(torch, step)
    _replay_and_check(torch, g, outs, want, "attention", between)


def test_decoder_block_graph_replay():
    """Block pre-attention stage, attention, post-attention stage and the
    backward in the reverse order, captured as one graph."""
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    from gemm_online_rmsnorm_amd.runner import BlockRun

    heads, seq_len = 2, 256
    d = heads * DH
    s = synth.BlockShape("graph decoder block", T=2 * seq_len, d=d, r=64, F=688, D=d, P=1,
                         seed=34)
    say(f"[graph] decoder block T={s.T} d={d} heads={heads}")
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials,
                   synth.make_inputs(s))
    ashape = lr.attn_shape(s.T, seq_len, heads, heads, DH)
    lse = torch.empty(heads, s.T, dtype=torch.float32, device="cuda")
    ws_f = torch.empty(lr.attention_workspace_bytes(ashape, False), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(lr.attention_workspace_bytes(ashape, True), dtype=torch.uint8,
                       device="cuda")

    def step():
        run.fwd(stage=lr.LR_STAGE_PRE_ATTN)
        Q, K, V = run.out["Q"], run.out["K"], run.out["V"]
        lr.attention_fwd(ashape, Q, K, V, run.O, lse, ws_f)
        run.fwd(stage=lr.LR_STAGE_POST_ATTN)
        run.bwd(stage=lr.LR_STAGE_POST_ATTN)
        lr.attention_bwd(ashape, Q, K, V, run.O, run.dO, lse, run.dQ, run.dK, run.dV, ws_b)
        run.bwd(stage=lr.LR_STAGE_PRE_ATTN)

    step()
    torch.cuda.synchronize()
    # O, dQ, dK, dV are intermediate here: written by attention inside the step.
    outs = _block_outputs(run) + [run.O, run.dQ, run.dK, run.dV, lse]
    want = [t.clone() for t in outs]
    for t in want:
        assert bool(torch.isfinite(t.float()).all())
    g = _capture(torch, step)
    other = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials,
                     synth.make_inputs(s, seed=35))
    _replay_and_check(torch, g, outs, want, "decoder block", other.step)
