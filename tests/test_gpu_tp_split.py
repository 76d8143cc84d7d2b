"""Parity of one rank's products under both tensor-parallel splits: every
forward, input-gradient and weight-gradient product of the comparison runs
through the library and is checked against the oracle's fp64 products."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import block as ob
from oracle import primitives as op
from oracle import share as osh
from tests.gpu_helpers import BF16_TOL, gpu_or_skip, rel_err, say

pytestmark = pytest.mark.gpu


def _h(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("split", ["vanilla", "bottleneck"])
def test_split_products_match_oracle(split):
    torch = gpu_or_skip()
    from gemm_online_rmsnorm_amd import tp_split as tps
    T, d, r, F, k = 264, 512, 256, 704, 4  # r / k = 64, d / k = 128, d_ff / k = 176
    gemms = (tps.vanilla_gemms if split == "vanilla" else tps.btp_gemms)(T, d, r, F, k)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for g in gemms:
        for label, layout, G, M, N, K in tps.products(g):
            say(f"[case] {split} {label} {layout} G={G} {M}x{N}x{K}")
            ops = tps.Operands(layout, G, M, N, K, gen)
            tps.run_product(layout, g, ops, M, N, K)
            torch.cuda.synchronize()
            xs = [_h(x) for x in ops.X]
            ws = [_h(w) for w in ops.W]
            if layout == "NT" and g.norm:
                gam = _h(ops.gamma)
                if g.partial:
                    ref, ss_ref = osh.norm_chunk_payload(gam, xs[0], ws[0])
                    assert rel_err(_h(ops.ss), ss_ref) <= 1e-5
                else:
                    ref, _, _ = ob.online_rmsnorm_matmul(xs[0], gam, ws[0], 1, g.d_norm, 1e-5)
                refs = [ref]
            elif layout == "NT" and g.swiglu:
                refs = op.grouped_gemm("NT", list(zip(xs, ws)), "swiglu")
            else:
                refs = op.grouped_gemm(layout, list(zip(xs, ws)))
            for y, ref in zip(ops.Y, refs):
                assert rel_err(_h(y), ref) <= BF16_TOL, label
