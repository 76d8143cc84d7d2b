"""The no-allocation Online RMSNorm GEMM (lr_online_rmsnorm_gemm_noalloc)
against the workspace variant (lr_online_rmsnorm_gemm), through the C ABI:
two calls in a row, the second with a smaller input, each compared with the
workspace variant on the same inputs. Both run the same kernels on the same
gamma-folded weights, so the outputs, RMS values and per-panel sums must be
bitwise equal (the parity bar of the path is max|a - b| / max|b| <= 1e-2 for
bf16 and 1e-5 for fp32; equality is stricter)."""
from __future__ import annotations

import pytest

from tests.gpu_helpers import gpu_or_skip, say

pytestmark = pytest.mark.gpu

# (label, T, d, N, panels, dtype): the first fills most of the scratch
# (3072 x 8192 bf16 = 48 MiB), the second is smaller and ragged.
CALLS = [("large", 2048, 8192, 3072, 2, "bf16"), ("small ragged", 300, 512, 200, 1, "bf16"),
         ("fp32", 130, 256, 96, 4, "f32")]


def _inputs(torch, T, d, N, dt, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    X = torch.randn(T, d, device="cuda", generator=g).to(dt)
    A = (torch.randn(N, d, device="cuda", generator=g) / d ** 0.5).to(dt)
    gamma = (1 + 0.1 * torch.randn(d, device="cuda", generator=g)).to(dt)
    return X, A, gamma


def test_noalloc_matches_workspace_variant_on_consecutive_calls():
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    for i, (label, T, d, N, P, dts) in enumerate(CALLS):
        dt = torch.bfloat16 if dts == "bf16" else torch.float32
        say(f"[case] no-alloc call {i}: {label} T={T} d={d} N={N} P={P} {dts}")
        X, A, gamma = _inputs(torch, T, d, N, dt, 100 + i)
        outs = []
        for fn in (lr.online_rmsnorm_gemm, lr.online_rmsnorm_gemm_noalloc):
            out = torch.full((T, N), float("nan"), device="cuda", dtype=dt)
            rms = torch.full((T,), float("nan"), device="cuda")
            ss = torch.full((P, T), float("nan"), device="cuda")
            fn(X, gamma, A, out, n_panels=P, rms_out=rms, ss_out=ss)
            torch.cuda.synchronize()
            outs.append((out, rms, ss))
        (o0, r0, s0), (o1, r1, s1) = outs
        assert torch.isfinite(o0.float()).all() and torch.isfinite(r0).all()
        for a, b, name in ((o1, o0, "out"), (r1, r0, "rms"), (s1, s0, "ss")):
            if not torch.equal(a, b):
                err = ((a.float() - b.float()).abs().max() / b.float().abs().max()).item()
                pytest.fail(f"{label}: {name} differs from the workspace variant ({err:.3e})")
    # beyond the scratch: rejected before anything is enqueued
    X, A, gamma = _inputs(torch, 64, 8192, 4104, torch.bfloat16, 7)
    out = torch.empty(64, 4104, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(lr.LRError) as e:
        lr.online_rmsnorm_gemm_noalloc(X, gamma, A, out)
    assert e.value.code == lr._lib.LR_ERR_WORKSPACE
