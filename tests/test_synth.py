"""Pins of the shared input generator (bf16 rounding and shapes)."""
from __future__ import annotations

import numpy as np
import torch

import synth


def test_bf16_round_to_nearest_even_known_values():
    x = np.array([1.0, -2.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20,
                  3.140625, 0.0], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    # 1+2^-8 is a tie between 0x3F80 and 0x3F81: even wins; 1+3*2^-8 ties
    # between 0x3F81 and 0x3F82: even wins; just above a tie rounds up.
    assert list(bits) == [0x3F80, 0xC000, 0x3F80, 0x3F82, 0x3F81, 0x4049, 0x0000]
    assert np.array_equal(synth.bf16_bits_to_f32(bits)[:2], np.array([1.0, -2.0], np.float32))


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-6, 6, 100000)).astype(np.float32)
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_inputs_shapes_and_distributions():
    s = synth.config(1)
    inp = synth.make_inputs(s)
    assert inp["X"].shape == (256, 256) and inp["B_g"].shape == (688, 64)
    assert inp["A_dn"].shape == (64, 688)
    assert abs(inp["A_q"].std() * np.sqrt(256) - 1) < 0.05
    assert abs(inp["A_dn"].std() * np.sqrt(688) - 1) < 0.05
    assert abs(inp["B_q"].std() * np.sqrt(64) - 1) < 0.05
    assert abs(inp["gamma1"].mean() - 1) < 0.02
    again = synth.make_inputs(s)
    assert all(np.array_equal(inp[k], again[k]) for k in inp)


def test_bf16_inputs_are_representable():
    s = synth.BlockShape("t", T=8, d=64, r=16, F=40, D=64, seed=3)
    inp = synth.make_inputs(s)
    for v in inp.values():
        assert np.array_equal(synth.round_to_bf16(v), v)


def test_configs_follow_r_equals_d_over_4():
    for n in (1, 2, 3, 4):
        s = synth.config(n)
        assert s.r * 4 == s.d
    s5 = synth.config(5)
    assert s5.D == 6656 and s5.d * 4 == s5.D and s5.r * 4 == s5.D
    assert s5.F * 4 == 17920
