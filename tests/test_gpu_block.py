"""Block forward + backward through the C ABI against the fp64 oracle, at
sizes the oracle finishes in seconds: several tiles, ragged tails, Online
RMSNorm panels, the rank-share mode and degenerate shapes. Also checks that
staged calls and repeated runs are bitwise identical."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import BF16_TOL, F32_TOL, ErrAcc, gpu_or_skip, say

pytestmark = pytest.mark.gpu

S = synth.BlockShape
CASES = {
    "tiny-fp32": synth.config(1),
    "tiny-fp32-P4": synth.config(1).replace(name="tiny-fp32-P4", P=4),
    "fp32-ragged": S("fp32-ragged", T=100, d=96, r=20, F=60, D=96, dtype="f32", seed=31),
    "bf16-ragged": S("bf16-ragged", T=300, d=320, r=80, F=424, D=320, seed=21),
    "bf16-P4": S("bf16-P4", T=264, d=512, r=128, F=344, D=512, P=4, seed=22),
    "bf16-share": S("bf16-share", T=200, d=192, r=192, F=320, D=768, partials=True,
                    fan_in_d=768, fan_in_F=1280, seed=23),
    "bf16-min": S("bf16-min", T=1, d=8, r=8, F=8, D=8, seed=24),
    "bf16-narrow": S("bf16-narrow", T=520, d=64, r=16, F=136, D=64, seed=25),
    # gate/up grids of at least 256 block-diagonal tiles of 256 x 128, ragged
    # in rows and columns, with K = r of two k-tiles and of one
    "bf16-gateup-r128": S("bf16-gateup-r128", T=4100, d=512, r=128, F=2112, D=512, seed=26),
    "bf16-gateup-r64": S("bf16-gateup-r64", T=4100, d=256, r=64, F=2104, D=256, seed=27),
    # ... and of at least 512 packed tiles of 160 x 128 (two per CU, the
    # tile of the 16384-token workloads), ragged in rows (100 of 160) and
    # columns (40 of 128)
    "bf16-gateup-packed-r128": S("bf16-gateup-packed-r128", T=4100, d=512, r=128, F=2600,
                                 D=512, seed=33),
    "bf16-gateup-packed-r64": S("bf16-gateup-packed-r64", T=4100, d=256, r=64, F=2600, D=256,
                                seed=34),
    # r a multiple of 32 but not of 64: gate/up tiles with k-tiles of 32,
    # dm on the general engine before the two-pair recompute tile
    "bf16-r96": S("bf16-r96", T=300, d=256, r=96, F=424, D=256, seed=32),
    # the split gate/up tiles (gate and up waves side by side) in both
    # directions: 192 rows with k-tiles of 64 (grids of 256 such tiles but
    # fewer of the larger ones), and 256 rows with k-tiles of 32 (r = 96)
    "bf16-split192": S("bf16-split192", T=3000, d=256, r=64, F=2048, D=256, seed=35),
    "bf16-split256-r96": S("bf16-split256-r96", T=4104, d=256, r=96, F=2056, D=256,
                           seed=36),
    # weight gradients of several shapes in one launch (dA_gu, dB_o, dA_o;
    # dA_qkv with dB_dn): with K split over per-problem partials (16 k-tiles)
    # and unsplit with ragged tiles (17 k-tiles, d and r not multiples of 256)
    "bf16-wgrad-group-split": S("bf16-wgrad-group-split", T=1024, d=1024, r=256, F=704,
                                D=1024, seed=28),
    "bf16-wgrad-group-ragged": S("bf16-wgrad-group-ragged", T=1088, d=1280, r=320, F=832,
                                 D=1280, seed=29),
}


def _run(s, inputs=None):
    from gemm_online_rmsnorm_amd.runner import BlockRun
    inputs = inputs if inputs is not None else synth.make_inputs(s)
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials, inputs)
    run.step()
    return run, inputs


def _compare(s, res, inputs, label):
    ref = oracle.run_fwd_bwd(inputs, D=s.D, eps=s.eps, n_panels=s.P, partials=s.partials)
    acc = ErrAcc()
    for k, v in ref.items():
        acc.add(k, res[k], v)
    missing = set(res) - set(ref)
    assert not missing, missing
    return acc.check(BF16_TOL if s.dtype == "bf16" else F32_TOL, label)


@pytest.mark.parametrize("name", list(CASES))
def test_block_parity(name):
    gpu_or_skip()
    s = CASES[name]
    say(f"[case] {name} T={s.T} d={s.d} r={s.r} F={s.F} D={s.D} P={s.P} {s.dtype}")
    run, inputs = _run(s)
    _compare(s, run.results(), inputs, name)


def test_stages_match_single_call_bitwise():
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    s = CASES["bf16-ragged"]
    run, inputs = _run(s)
    full = run.results()
    # zero the outputs, then run the stages in a trainer's order
    for t in list(run.out.values()) + list(run.saved.values()) + list(run.grads.values()):
        t.zero_()
    run.dX.zero_()
    run.dO.zero_()
    run.fwd(lr.LR_STAGE_PRE_ATTN)
    run.fwd(lr.LR_STAGE_POST_ATTN)
    run.bwd(lr.LR_STAGE_POST_ATTN)
    run.bwd(lr.LR_STAGE_PRE_ATTN)
    torch.cuda.synchronize()
    staged = run.results()
    for k in full:
        assert np.array_equal(full[k], staged[k]), k


def test_runs_are_bitwise_deterministic():
    gpu_or_skip()
    s = CASES["bf16-P4"]
    run, inputs = _run(s)
    a = run.results()
    run.step()
    b = run.results()
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_pre_attention_stage_leaves_post_outputs_untouched():
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    s = CASES["bf16-narrow"]
    from gemm_online_rmsnorm_amd.runner import BlockRun
    inputs = synth.make_inputs(s)
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials, inputs)
    run.out["Y"].fill_(7.0)
    run.fwd(lr.LR_STAGE_PRE_ATTN)
    torch.cuda.synchronize()
    assert bool(torch.all(run.out["Y"] == 7.0))
    ref = oracle.run_fwd_bwd(inputs, D=s.D, eps=s.eps, backward=False)
    acc = ErrAcc()
    res = run.results()
    for k in ("Q", "K", "V", "qkv_r", "rms1"):
        acc.add(k, res[k], ref[k])
    acc.check(BF16_TOL, "pre-attention stage")
