"""Low-rank activation checkpointing on the GPU: the d-wide activations the
backward recomputes from the saved r-wide ones equal, bit for bit, those the
forward computed (project page, "Three supporting changes": checkpointing
without communication recomputes h and the MLP's g, u from q_r ... d_r).

The forward's h = X + o_r B_o^T and m = SiLU(g) * u stay in the forward
workspace; the backward recomputes both into its own workspace (g and u only
inside the tile that forms m, dg and du, so they are checked through m).
Both are located with lr_block_workspace_tensor. The backward workspace is
filled with NaN first, so a stale value cannot pass. The forward's h and m
are also compared with the oracle's tape (they are the right tensors)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import BF16_TOL, F32_TOL, gpu_or_skip, rel_err, say

pytestmark = pytest.mark.gpu

S = synth.BlockShape
CASES = {
    "tiny-fp32": synth.config(1),
    "fp32-ragged": S("fp32-ragged", T=100, d=96, r=20, F=60, D=96, dtype="f32", seed=41),
    "bf16-ragged": S("bf16-ragged", T=300, d=320, r=80, F=424, D=320, seed=42),
    # r a multiple of 32 but not of 64: the forward's gate/up tile and the
    # backward's three-pair recompute tile (dm in the same tile) differ
    "bf16-r96": S("bf16-r96", T=300, d=256, r=96, F=424, D=256, seed=45),
    # large tiles: the 256 x 256 residual tile and the gate/up tile of the
    # 16384-token workloads, with partial row and column tiles
    "bf16-large-tiles": S("bf16-large-tiles", T=1000, d=1024, r=256, F=2752, D=1024, P=2,
                          seed=43),
    "bf16-share": S("bf16-share", T=200, d=192, r=192, F=320, D=768, partials=True,
                    fan_in_d=768, fan_in_F=1280, seed=44),
    # the gate/up tiles of larger grids: packed 160 x 128 (the 16384-token
    # workloads' tile), the 192-row split tile and the 256-row split tile
    "bf16-packed": S("bf16-packed", T=4100, d=256, r=64, F=2600, D=256, seed=46),
    "bf16-split192": S("bf16-split192", T=3000, d=256, r=64, F=2048, D=256, seed=47),
    "bf16-split256-r96": S("bf16-split256-r96", T=4104, d=256, r=96, F=2056, D=256, seed=48),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_recompute_equals_forward_bitwise(name):
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    from gemm_online_rmsnorm_amd.runner import BlockRun
    s = CASES[name]
    say(f"[case] checkpoint {name} T={s.T} d={s.d} r={s.r} F={s.F} D={s.D} P={s.P} {s.dtype}")
    inputs = synth.make_inputs(s)
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials, inputs)
    run.fwd()
    torch.cuda.synchronize()
    fwd = {w: lr.workspace_tensor(run.shape, run.ws_f, False, w).clone()
           for w in (lr.LR_WS_H, lr.LR_WS_M)}
    run.ws_b.fill_(0xFF)  # NaN in bf16 and fp32
    run.bwd()
    torch.cuda.synchronize()
    for w, label in ((lr.LR_WS_H, "h"), (lr.LR_WS_M, "m")):
        bwd = lr.workspace_tensor(run.shape, run.ws_b, True, w)
        assert bwd.shape == fwd[w].shape
        assert torch.isfinite(bwd.float()).all(), label
        same = torch.equal(bwd.view(torch.int16 if bwd.element_size() == 2 else torch.int32),
                           fwd[w].view(torch.int16 if bwd.element_size() == 2 else torch.int32))
        if not same:
            diff = (bwd.float() - fwd[w].float()).abs().max().item()
            pytest.fail(f"{name}: recomputed {label} differs from the forward's (max {diff:.3e})")
    # The forward's values are the block's h and m.
    W = {k: inputs[k].astype(np.float64) for k in oracle.blocked._WEIGHTS}
    X, O = inputs["X"].astype(np.float64), inputs["O"].astype(np.float64)
    if s.partials:
        tape = oracle.share_forward(W, X, O, s.D, s.eps)
        h_ref = X + tape["o_r"] @ W["B_o"].T
        m_ref = oracle.silu(tape["g_r"] @ W["B_g"].T) * (tape["u_r"] @ W["B_u"].T)
    else:
        tape = oracle.block_forward(W, X, O, s.D, s.eps, tape=True)
        h_ref, m_ref = tape["h"], tape["m"]
    tol = BF16_TOL if s.dtype == "bf16" else F32_TOL
    for w, ref, label in ((lr.LR_WS_H, h_ref, "h"), (lr.LR_WS_M, m_ref, "m")):
        e = rel_err(fwd[w].float().cpu().numpy(), ref)
        say(f"  forward {label} vs oracle: {e:.2e}")
        assert e <= tol, (label, e)
