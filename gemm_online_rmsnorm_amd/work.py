"""Algorithmic work of every kernel launch of one block step.

For each launch the library makes (keyed by the name its measurement hook
records), the FLOP count (a multiply-add is 2 FLOP) and the algorithmic HBM
bytes: every operand read once and every output written once, in the
storage type. The fp32 weight gradients count 4 bytes per element. These
are the numerators of the roofline figures; the denominators are measured.
"""
from __future__ import annotations


def kernel_work(T: int, d: int, r: int, F: int, elem: int = 2, partials: bool = False,
                n_panels: int = 1) -> dict[str, tuple[float, float]]:
    e = elem
    W = {}

    def g(name, M, N, K, extra_in=0, out_elem=None, n_in_mats=None):
        """GEMM M x N x K: flops and bytes (X, W read once; Y written once)."""
        oe = e if out_elem is None else out_elem
        W[name] = (2.0 * M * N * K, e * (M * K + N * K) + oe * M * N + extra_in)

    # forward
    W["fold gamma1"] = (0.0, e * (2 * 3 * r * d + d))
    g("QKV Online RMSNorm GEMM", T, 3 * r, d, extra_in=4 * T * (n_panels + 1))
    if partials:
        W["QKV finalize"] = (0.0, e * 2 * T * 3 * r + 8 * T)
    W["QKV grouped up-projection"] = (3 * 2.0 * T * d * r, 3 * e * (T * r + d * r + T * d))
    g("O down-projection", T, r, d)
    g("O up-projection + residual", T, d, r, extra_in=e * T * d)
    W["fold gamma2"] = (0.0, e * (2 * 2 * r * d + d))
    W["fold gamma1, gamma2"] = (0.0, e * (2 * 5 * r * d + 2 * d))
    g("gate/up Online RMSNorm GEMM", T, 2 * r, d, extra_in=4 * T * (n_panels + 1))
    if partials:
        W["gate/up finalize"] = (0.0, e * 2 * T * 2 * r + 8 * T)
    W["gate/up up-projection + SwiGLU"] = (2 * 2.0 * T * F * r,
                                           e * (2 * T * r + 2 * F * r + T * F))
    g("down-projection", T, r, F)
    g("down up-projection + residual", T, d, r, extra_in=e * T * d)
    # backward
    # transposed copies of the weights the data-gradient products multiply by
    W["transpose B_dn, A_dn, B_g, B_u, A_gu, B_o, A_o"] = (0.0, 2 * e * r * (5 * d + 3 * F))
    W["transpose B_q, B_k, B_v, A_qkv"] = (0.0, 2 * e * 6 * r * d)
    g("dB_dn", d, r, T, out_elem=4)
    g("dd_r", T, r, d)
    if e == 2:
        # dm = dd_r A_dn, then g, u recomputed with m, dg, du from dm in the epilogue
        g("dm = dd_r A_dn", T, F, r)
        W["SwiGLU recompute + backward"] = (2 * 2.0 * T * F * r,
                                            e * (2 * T * r + 2 * F * r + 4 * T * F))
    else:
        # fp32: one tile with three accumulators (g, u, dm)
        W["SwiGLU recompute + backward"] = (3 * 2.0 * T * F * r,
                                            e * (3 * T * r + 3 * F * r + 3 * T * F))
    g("dA_dn", r, F, T, out_elem=4)
    W["dB_g, dB_u"] = (2 * 2.0 * F * r * T, 2 * (e * (T * F + T * r) + 4 * F * r))
    W["dgu_r"] = (2 * 2.0 * T * r * F, 2 * e * (T * F + F * r + T * r) + 4 * T)
    W["row dot 2"] = (2.0 * T * 2 * r, e * 2 * T * 2 * r + 8 * T)
    g("recompute h", T, d, r, extra_in=e * T * d)
    g("RMSNorm-2 backward", T, d, 2 * r, extra_in=2 * e * T * d + 4 * T + e * d)
    W["dgamma2 column sum"] = (0.0, 4 * ((T + 255) // 256) * d + 4 * d)
    g("dA_gu", 2 * r, d, T, out_elem=4, extra_in=e * d)
    g("dB_o", d, r, T, out_elem=4)
    g("do_r", T, r, d)
    g("dA_o", r, d, T, out_elem=4)
    g("dO", T, d, r)
    W["dB_q, dB_k, dB_v"] = (3 * 2.0 * d * r * T, 3 * (e * (T * d + T * r) + 4 * d * r))
    W["dqkv_r"] = (3 * 2.0 * T * r * d, 3 * e * (T * d + d * r + T * r) + 4 * T)
    W["row dot 1"] = (2.0 * T * 3 * r, e * 2 * T * 3 * r + 8 * T)
    g("RMSNorm-1 backward", T, d, 3 * r, extra_in=2 * e * T * d + 4 * T + e * d)
    W["dgamma1 column sum"] = (0.0, 4 * ((T + 255) // 256) * d + 4 * d)
    g("dA_qkv", 3 * r, d, T, out_elem=4, extra_in=e * d)
    # weight gradients that run together in one launch
    for name, parts in (("dA_gu, dB_o, dA_o", ("dA_gu", "dB_o", "dA_o")),
                        ("dA_qkv, dB_dn", ("dA_qkv", "dB_dn"))):
        W[name] = (sum(W[k][0] for k in parts), sum(W[k][1] for k in parts))
    return W


# Kernels bounded by HBM bandwidth rather than by the matrix cores (the
# fixed-order sums of split-K weight-gradient slices are named
# "<weight gradient> split-K sum").
MEMORY_BOUND = ("fold gamma1", "fold gamma2", "fold gamma1, gamma2", "fold gamma",
                "QKV finalize", "gate/up finalize",
                "row dot 1", "row dot 2", "dgamma1 column sum", "dgamma2 column sum",
                "transpose B_dn, A_dn, B_g, B_u, A_gu, B_o, A_o", "transpose B_q, B_k, B_v, A_qkv")


def is_memory_bound(name: str) -> bool:
    return name in MEMORY_BOUND or name.endswith("split-K sum")
