"""Full-size parity: the 16384-token bf16 workloads (1B, 7B, 13B with four
Online RMSNorm panels, and the 30B rank share), run in the launch
configuration bench.py times, compared element by element in full against
the row-blocked fp64 oracle (every output, saved activation, partial and
gradient)."""
from __future__ import annotations

import time

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import BF16_TOL, ErrAcc, gpu_or_skip, say

pytestmark = pytest.mark.gpu

WGRADS = ("dgamma1", "dgamma2", "dA_qkv", "dB_q", "dB_k", "dB_v", "dA_o", "dB_o", "dA_gu",
          "dB_g", "dB_u", "dA_dn", "dB_dn")


# Ragged variants of the 16384-token shapes: the token count leaves a
# partial 256-row tile whose last 16-row band is half full, and d, r and d_ff
# leave partial column tiles, so the large tiles' epilogues (band inputs,
# stores, column sums) and the split gate/up tile run with rows and columns
# past the matrix. All sizes stay multiples of 64.
RAGGED = {
    "1B-ragged-P2": synth.config(2).replace(name="1B-ragged-P2", T=16008, d=1920, r=448,
                                            F=5568, D=1920, P=2, heads=16),
    "30B-rank0of4-ragged": synth.config(5).replace(name="30B-rank0of4-ragged", T=16008),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 4, 5] + list(RAGGED))
def test_full_workload_parity(cfg):
    torch = gpu_or_skip()
    from gemm_online_rmsnorm_amd.runner import BlockRun
    s = RAGGED[cfg] if isinstance(cfg, str) else synth.config(cfg)
    say(f"[case] full workload {cfg}: {s.name} T={s.T} d={s.d} r={s.r} F={s.F} D={s.D} P={s.P}")
    t0 = time.time()
    inputs = synth.make_inputs(s)
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials, inputs,
                   heads=s.heads)
    run.step()
    res = run.results(host_dtype=np.float32)
    del run
    torch.cuda.empty_cache()
    say(f"  gpu done in {time.time() - t0:.1f}s; running the oracle")
    acc = ErrAcc()

    def on_rows(sel, loc):
        for k, v in loc.items():
            if k.startswith("ss_panels"):
                acc.add(k, res[k][:, sel].T, v)
            else:
                acc.add(k, res[k][sel], v)

    ref = oracle.run_fwd_bwd(inputs, D=s.D, eps=s.eps, n_panels=s.P, partials=s.partials,
                             row_block=2048, on_rows=on_rows)
    for k in WGRADS:
        acc.add(k, res[k], ref[k])
    say(f"  oracle done at {time.time() - t0:.1f}s")
    errs = acc.check(BF16_TOL, s.name)
    assert len(errs) >= 23
    assert np.isfinite(list(errs.values())).all()
