"""Host logic of the tensor-parallel split comparison (CPU only)."""
from __future__ import annotations

from gemm_online_rmsnorm_amd import tp_split as tps

SHAPE = dict(T=16384, d=4096, r=1024, F=11008)  # LLaMA-7B, the page's volume table


def test_splits_do_the_same_work():
    """Both splits give one rank the same multiply-adds, product by product."""
    for k in (2, 4, 8):
        van = tps.vanilla_gemms(**SHAPE, k=k)
        btp = tps.btp_gemms(**SHAPE, k=k)
        assert [g.name.split(" (")[0].replace(" + SwiGLU", "") for g in van] == \
               [g.name.split(" (")[0].replace(" + SwiGLU", "") for g in btp]
        for a, b in zip(van, btp):
            assert a.flops() == b.flops()
        full = 2.0 * SHAPE["T"] * SHAPE["r"] * (11 * SHAPE["d"] + 3 * SHAPE["F"])
        assert sum(g.flops() for g in van) * k == full


def test_allreduce_volume_matches_the_page_table():
    """BOOST project page, volume table: vanilla low-rank TP sends 5bsd +
    2bsd_ff per block and pass (5.19x full-rank TP's 2bsd at LLaMA-7B),
    BOOST 7bsr (0.88x)."""
    d, r, F = SHAPE["d"], SHAPE["r"], SHAPE["F"]
    full = 2 * d
    assert round(tps.allreduce_values_per_token("vanilla", d, r, F) / full, 2) == 5.19
    assert round(tps.allreduce_values_per_token("btp", d, r, F) / full, 2) == 0.88


def test_backward_products_are_the_transposed_shapes():
    g = tps.Gemm("x", False, 3, 100, 60, 40)
    (f, lf, *sf), (dx, ldx, *sdx), (dw, ldw, *sdw) = tps.products(g)
    assert (lf, ldx, ldw) == ("NT", "NN", "TN")
    assert sf == [3, 100, 60, 40] and sdx == [3, 100, 40, 60] and sdw == [3, 60, 40, 100]
    # the same multiply-adds in all three
    for _, _, G, M, N, K in tps.products(g):
        assert G * M * N * K == 3 * 100 * 60 * 40
