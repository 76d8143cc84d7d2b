"""Parity of the standalone entry points (grouped low-rank GEMM, Online
RMSNorm GEMM) with the oracle, on ragged shapes spanning several tiles."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import block as ob
from oracle import primitives as op
from oracle import share as osh
from tests.gpu_helpers import BF16_TOL, F32_TOL, gpu_or_skip, rel_err, say

pytestmark = pytest.mark.gpu


def _rand(rng, shape, dtype, scale=1.0):
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return synth.round_to_bf16(v) if dtype == "bf16" else v


def _dev(torch, a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


LAYOUT = {"NT": 0, "NN": 1, "TN": 2}


# bf16 products whose K is a multiple of 64 (32 for the gate/up pair) and
# whose N is a multiple of 8 run on the pipelined engine; the others on the
# general one. Each test covers both.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("G", [1, 3])
@pytest.mark.parametrize("K", [136, 128])
def test_grouped_gemm_layouts(dtype, layout, G, K):
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    rng = np.random.default_rng(100 * (dtype == "bf16") + 10 * LAYOUT[layout] + G + K)
    M, N = 296, 200
    xs = (K, M) if layout == "TN" else (M, K)
    ws = (N, K) if layout == "NT" else (K, N)
    pairs_h = [(_rand(rng, xs, dtype), _rand(rng, ws, dtype, 1 / np.sqrt(K))) for _ in range(G)]
    odt = torch.float32 if (layout == "TN" or dtype == "f32") else torch.bfloat16
    ys = [torch.empty(M, N, dtype=odt, device="cuda") for _ in range(G)]
    pairs = [dict(M=M, N=N, K=K, X=_dev(torch, x, dtype), W=_dev(torch, w, dtype), Y=y)
             for (x, w), y in zip(pairs_h, ys)]
    lr.grouped_lowrank_gemm(pairs, lr.LR_BF16 if dtype == "bf16" else lr.LR_F32,
                            LAYOUT[layout], lr.LR_EPI_NONE)
    torch.cuda.synchronize()
    ref = op.grouped_gemm(layout, pairs_h)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    for y, r in zip(ys, ref):
        e = rel_err(_host(y), r)
        say(f"grouped {layout} G={G} {dtype}: {e:.2e}")
        assert e <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["NT", "NN"])
@pytest.mark.parametrize("shape", [(264, 136, 72), (264, 136, 64), (4088, 4040, 64),
                                   (4360, 4040, 64)])
def test_gemm_epilogues(dtype, layout, shape):
    """Plain, residual and row-scale epilogues; the last two shapes run
    256 x 256 tiles with a partial last row band and a partial last column
    tile, the last one 288 of them, so that the persistent workgroups (one
    per CU) run a second tile, ragged, after a first one."""
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    rng = np.random.default_rng(7 + shape[2])
    M, N, K = shape
    dl = lr.LR_BF16 if dtype == "bf16" else lr.LR_F32
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    x = _rand(rng, (M, K), dtype)
    w = _rand(rng, (N, K) if layout == "NT" else (K, N), dtype, 1 / np.sqrt(K))
    res = _rand(rng, (M, N), dtype)
    rs = np.abs(rng.standard_normal(M).astype(np.float32)) + 0.5
    odt = torch.bfloat16 if dtype == "bf16" else torch.float32
    X, Wd = _dev(torch, x, dtype), _dev(torch, w, dtype)
    # residual
    y = torch.empty(M, N, dtype=odt, device="cuda")
    lr.grouped_lowrank_gemm([dict(M=M, N=N, K=K, X=X, W=Wd, Y=y, aux=_dev(torch, res, dtype))],
                            dl, LAYOUT[layout], lr.LR_EPI_ADD_RESIDUAL)
    # row scale
    y2 = torch.empty(M, N, dtype=odt, device="cuda")
    rsd = torch.from_numpy(rs).cuda()
    lr.grouped_lowrank_gemm([dict(M=M, N=N, K=K, X=X, W=Wd, Y=y2, aux=rsd)], dl, LAYOUT[layout],
                            lr.LR_EPI_ROW_SCALE)
    # plain
    y3 = torch.empty(M, N, dtype=odt, device="cuda")
    lr.grouped_lowrank_gemm([dict(M=M, N=N, K=K, X=X, W=Wd, Y=y3)], dl, LAYOUT[layout],
                            lr.LR_EPI_NONE)
    torch.cuda.synchronize()
    say(f"[case] epilogues {layout} {dtype} {shape}")
    assert rel_err(_host(y), op.grouped_gemm(layout, [(x, w)], "residual", res)[0]) <= tol
    assert rel_err(_host(y2), op.grouped_gemm(layout, [(x, w)], "row_scale", rs)[0]) <= tol
    assert rel_err(_host(y3), op.grouped_gemm(layout, [(x, w)])[0]) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 344, 80), (300, 344, 96), (4104, 2056, 96),
                                   (4104, 2056, 128)])
def test_swiglu_pair(dtype, shape):
    """The last two shapes run the split gate/up tile (256 rows x 128 gate +
    128 up columns) with partial last row and column tiles, over an odd and
    an even number of k-tiles."""
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    rng = np.random.default_rng(11 + shape[2])
    M, N, K = shape
    xg, xu = _rand(rng, (M, K), dtype), _rand(rng, (M, K), dtype)
    wg = _rand(rng, (N, K), dtype, 1 / np.sqrt(K))
    wu = _rand(rng, (N, K), dtype, 1 / np.sqrt(K))
    odt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.empty(M, N, dtype=odt, device="cuda")
    y1 = torch.empty(M, N, dtype=odt, device="cuda")
    pairs = [dict(M=M, N=N, K=K, X=_dev(torch, xg, dtype), W=_dev(torch, wg, dtype), Y=y),
             dict(M=M, N=N, K=K, X=_dev(torch, xu, dtype), W=_dev(torch, wu, dtype), Y=y1)]
    lr.grouped_lowrank_gemm(pairs, lr.LR_BF16 if dtype == "bf16" else lr.LR_F32, 0,
                            lr.LR_EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    ref = op.grouped_gemm("NT", [(xg, wg), (xu, wu)], "swiglu")[0]
    assert rel_err(_host(y), ref) <= (BF16_TOL if dtype == "bf16" else F32_TOL)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_online_rmsnorm_gemm(dtype, P):
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    rng = np.random.default_rng(100 + P)
    T, d, N = 300, 512, 136
    D = d
    x = _rand(rng, (T, d), dtype) * np.float32(1.0)
    x[5] *= np.float32(8.0)          # rows of very different scale
    x[7] *= np.float32(0.125)
    gamma = 1 + 0.1 * _rand(rng, (d,), "f32")
    gamma = synth.round_to_bf16(gamma) if dtype == "bf16" else gamma
    A = _rand(rng, (N, d), dtype, 1 / np.sqrt(d))
    odt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty(T, N, dtype=odt, device="cuda")
    rms = torch.empty(T, dtype=torch.float32, device="cuda")
    ss = torch.empty(P, T, dtype=torch.float32, device="cuda")
    Xd = _dev(torch, x, dtype)
    lr.online_rmsnorm_gemm(Xd, _dev(torch, gamma, dtype), _dev(torch, A, dtype), out,
                           n_panels=P, d_norm=D, eps=1e-5, rms_out=rms, ss_out=ss)
    # partial mode: unscaled product and the total sum of squares
    outp = torch.empty(T, N, dtype=odt, device="cuda")
    ssp = torch.empty(T, dtype=torch.float32, device="cuda")
    lr.online_rmsnorm_gemm(Xd, _dev(torch, gamma, dtype), _dev(torch, A, dtype), outp,
                           n_panels=1, d_norm=4 * D, eps=1e-5, ss_out=ssp, emit_partial=True)
    torch.cuda.synchronize()
    x64, g64, A64 = (v.astype(np.float64) for v in (x, gamma, A))
    ref, rms_ref, ss_ref = ob.online_rmsnorm_matmul(x64, g64, A64, P, D, 1e-5)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    e = rel_err(_host(out), ref)
    abs_err = np.abs(_host(out) - ref)
    say(f"ORMS {dtype} P={P}: rel {e:.2e}, max abs {abs_err.max():.2e}, mean abs {abs_err.mean():.2e}")
    assert e <= tol
    assert rel_err(_host(rms), rms_ref) <= 1e-5
    assert rel_err(_host(ss), ss_ref) <= 1e-5
    P_ref, ss_tot_ref = osh.norm_chunk_payload(g64, x64, A64)
    assert rel_err(_host(outp), P_ref) <= tol
    assert rel_err(_host(ssp), ss_tot_ref) <= 1e-5


def test_grouped_gemm_workspace_split_k():
    """The workspace variant of the grouped GEMM on a weight-gradient shape
    whose output grid is small (K split into fp32 partial slices): oracle
    parity and bitwise-identical repeats."""
    torch = gpu_or_skip()
    import gemm_online_rmsnorm_amd as lr
    rng = np.random.default_rng(21)
    M, N, K, G = 520, 264, 8192, 2
    pairs_h = [(_rand(rng, (K, M), "bf16"), _rand(rng, (K, N), "bf16", 1 / np.sqrt(K)))
               for _ in range(G)]
    ys = [torch.empty(M, N, dtype=torch.float32, device="cuda") for _ in range(G)]
    pairs = [dict(M=M, N=N, K=K, X=_dev(torch, x, "bf16"), W=_dev(torch, w, "bf16"), Y=y)
             for (x, w), y in zip(pairs_h, ys)]
    nb = lr.grouped_lowrank_gemm_workspace_bytes(pairs, lr.LR_BF16, lr.LR_LAYOUT_TN)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    lr.grouped_lowrank_gemm(pairs, lr.LR_BF16, lr.LR_LAYOUT_TN, lr.LR_EPI_NONE, ws=ws)
    torch.cuda.synchronize()
    first = [y.clone() for y in ys]
    ref = op.grouped_gemm("TN", pairs_h)
    for y, r in zip(ys, ref):
        e = rel_err(_host(y), r)
        say(f"grouped TN split-K ({nb} B workspace): {e:.2e}")
        assert e <= BF16_TOL
    lr.grouped_lowrank_gemm(pairs, lr.LR_BF16, lr.LR_LAYOUT_TN, lr.LR_EPI_NONE, ws=ws)
    torch.cuda.synchronize()
    for y, f in zip(ys, first):
        assert torch.equal(y, f)
