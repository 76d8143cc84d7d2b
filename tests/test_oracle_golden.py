"""Pins of the oracle against numbers the BOOST pages print."""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import share as osh
from tests.oracle_helpers import small_problem

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _payload_widths(r=4, d=16, F=24):
    """Widths of the r-wide all-reduce payloads one rank's forward emits."""
    s, W, f = small_problem(T=3, d=d, r=r, F=F, seed=21)
    gen = osh._forward_steps(W, f["X"], f["O"], s.D, 1e-5)
    widths = []
    payload = next(gen)
    try:
        while True:
            # the r-wide partial is the first item; a norm chunk adds a [T] ss
            widths.append((payload[0].shape[1], len(payload) - 1))
            payload = gen.send(payload)
    except StopIteration:
        pass
    return widths


def test_allreduce_volume_is_7r_per_token():
    g = _load("allreduce_volume_table.json")
    r = 4
    widths = _payload_widths(r=r)
    # chunks: QKV (3r + ss), O (r), gate+up (2r + ss), down (r)
    assert widths == [(3 * r, 1), (r, 0), (2 * r, 1), (r, 0)]
    per_token = sum(w for w, _ in widths)
    assert per_token == 7 * r
    L = g["llama7b"]
    ratio_boost = 7 * L["r"] / (2 * L["d"])
    ratio_vanilla = (5 * L["d"] + 2 * L["d_ff"]) / (2 * L["d"])
    assert round(ratio_boost, 2) == g["printed_ratio_vs_full_rank"]["boost"]
    assert round(ratio_vanilla, 2) == g["printed_ratio_vs_full_rank"]["vanilla_low_rank_tp"]


def test_precision_fixture_is_consistent_with_tolerances():
    """The parity gates (1e-5 fp32, 1e-2 bf16, relative to the max) sit
    above the pages' Online RMSNorm error for O(1) outputs."""
    g = _load("online_rmsnorm_precision.json")
    assert g["fp32"]["max_abs"] < 1e-5
    assert g["bf16"]["max_abs"] < 1e-1 and g["bf16"]["mean_abs"] < 1e-2
    assert np.isfinite(g["bf16"]["max_abs"])
