"""Seeded synthetic inputs for the low-rank decoder-block linear stack.

This module is shared by the tests, the benchmark and the smoke check. It
holds workload shapes, seeded random draws and the float32 -> bfloat16
round-to-nearest-even used to make the draws representable in bf16. It holds
none of the block's arithmetic (no norm, no matmul, no activation): the GPU
library and the CPU oracle each implement that on their own.

Workloads (BOOST project page, "Results": LLaMA-2-style models, micro-batch 4,
sequence length 4096, so 16384 tokens per step; the low-rank factorisation
uses r = d/4, "Move the chunk boundary to the bottleneck"):

  1  tiny fp32 block        T=256   d=256  r=64   F=688   (parity only)
  2  1B-shape bf16 block    T=16384 d=2048 r=512  F=5632
  3  7B-shape bf16 block    T=16384 d=4096 r=1024 F=11008
  4  13B-shape bf16 block   T=16384 d=5120 r=1280 F=13824, Online RMSNorm
                            over 4 K-panels of 1280 columns
  5  30B-shape rank share   rank 0 of 4: d=6656/4=1664 columns of the
                            residual stream, r=1664, F=17920/4=4480, the RMS
                            divisor is the global width 6656, and the block
                            emits its unreduced r-wide partial sums

Value distributions: X, O, dY, dQ, dK, dV ~ N(0,1); gamma = 1 + 0.1 N(0,1);
down-projections A ~ N(0, 1/fan_in) (fan_in = d, or d_ff for the MLP's
down-projection); up-projections B ~ N(0, 1/r). For the rank share the fan-in
is the global one (the slices are slices of the global weights).
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "BlockShape",
    "CONFIGS",
    "config",
    "make_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "round_to_bf16",
    "INPUT_ORDER",
    "WEIGHT_SHAPES",
]


@dataclasses.dataclass(frozen=True)
class BlockShape:
    """One workload: the sizes one GPU holds and how its inputs are drawn."""

    name: str
    T: int               # tokens (micro-batch x sequence)
    d: int               # hidden width held by this GPU
    r: int               # bottleneck rank
    F: int               # MLP width (d_ff) held by this GPU
    D: int               # RMS divisor: the global hidden width
    P: int = 1           # Online RMSNorm K-panels
    heads: int = 1       # layout information only; the linear stack ignores it
    dtype: str = "bf16"  # "bf16" or "f32"
    seed: int = 0
    partials: bool = False   # emit unreduced r-wide partial sums (rank share)
    fan_in_d: int = 0        # fan-in used for A ~ N(0, 1/fan_in); 0 = d
    fan_in_F: int = 0        # fan-in used for A_dn; 0 = F
    eps: float = 1e-5

    @property
    def fan_d(self) -> int:
        return self.fan_in_d or self.d

    @property
    def fan_F(self) -> int:
        return self.fan_in_F or self.F

    def replace(self, **kw) -> "BlockShape":
        return dataclasses.replace(self, **kw)

    # Algorithmic work per token (multiply-adds counted as 2 FLOP).
    def fwd_flop_per_token(self) -> int:
        return 2 * self.r * (11 * self.d + 3 * self.F)

    def bwd_flop_per_token(self) -> int:
        return 4 * self.r * (11 * self.d + 3 * self.F)

    def recompute_flop_per_token(self) -> int:
        # g and u (two r->F up-projections) and h (one r->d up-projection)
        return 2 * self.r * (2 * self.F + self.d)


CONFIGS: dict[int, BlockShape] = {
    1: BlockShape("tiny-fp32", T=256, d=256, r=64, F=688, D=256, P=1, heads=4,
                  dtype="f32", seed=0),
    2: BlockShape("1B-bf16", T=16384, d=2048, r=512, F=5632, D=2048, P=1,
                  heads=16, seed=1),
    3: BlockShape("7B-bf16", T=16384, d=4096, r=1024, F=11008, D=4096, P=1,
                  heads=32, seed=2),
    4: BlockShape("13B-bf16-P4", T=16384, d=5120, r=1280, F=13824, D=5120, P=4,
                  heads=40, seed=3),
    5: BlockShape("30B-rank0of4-bf16", T=16384, d=1664, r=1664, F=4480, D=6656,
                  P=1, heads=13, seed=4, partials=True, fan_in_d=6656,
                  fan_in_F=17920),
}


def config(n: int) -> BlockShape:
    return CONFIGS[n]


# Draw order of the seeded generator; every consumer draws in this order.
INPUT_ORDER = (
    "X", "O", "gamma1", "gamma2",
    "A_q", "A_k", "A_v", "B_q", "B_k", "B_v",
    "A_o", "B_o", "A_g", "A_u", "B_g", "B_u", "A_dn", "B_dn",
    "dY", "dQ", "dK", "dV",
)


def WEIGHT_SHAPES(s: BlockShape) -> dict[str, tuple[int, ...]]:
    """Weights are stored [out, in] row-major (y = x @ W.T)."""
    d, r, F = s.d, s.r, s.F
    return {
        "gamma1": (d,), "gamma2": (d,),
        "A_q": (r, d), "A_k": (r, d), "A_v": (r, d),
        "B_q": (d, r), "B_k": (d, r), "B_v": (d, r),
        "A_o": (r, d), "B_o": (d, r),
        "A_g": (r, d), "A_u": (r, d),
        "B_g": (F, r), "B_u": (F, r),
        "A_dn": (r, F), "B_dn": (d, r),
    }


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs are not expected (all draws are finite).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return out.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _std(s: BlockShape, name: str) -> float:
    if name.startswith("A_dn"):
        return 1.0 / np.sqrt(s.fan_F)
    if name.startswith("A_"):
        return 1.0 / np.sqrt(s.fan_d)
    if name.startswith("B_"):
        return 1.0 / np.sqrt(s.r)
    return 1.0


def make_inputs(s: BlockShape, seed: int | None = None) -> dict[str, np.ndarray]:
    """Seeded inputs of one workload as float32 arrays.

    For bf16 workloads every value is already bf16-representable, so the GPU
    side takes the upper 16 bits and the oracle widens the same values to
    float64 exactly.
    """
    rng = np.random.default_rng(s.seed if seed is None else seed)
    shapes = WEIGHT_SHAPES(s)
    out: dict[str, np.ndarray] = {}
    for name in INPUT_ORDER:
        if name in ("X", "O", "dY", "dQ", "dK", "dV"):
            shape = (s.T, s.d)
        else:
            shape = shapes[name]
        v = rng.standard_normal(shape, dtype=np.float32)
        if name.startswith("gamma"):
            v = np.float32(1.0) + np.float32(0.1) * v
        else:
            sd = _std(s, name)
            if sd != 1.0:
                v *= np.float32(sd)
        if s.dtype == "bf16":
            v = round_to_bf16(v)
        out[name] = v
    return out


# ---------------------------------------------------------------------------
# Attention core (causal RoPE attention between the block's Q, K, V and O).
# Shapes: LLaMA-2-7B has 32 heads of 128 (multi-head, 32 key/value heads);
# the grouped-query case uses 8 key/value heads for 32 query heads.
# Value distributions: Q, K, V, dO ~ N(0, 1), rounded to bf16.
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class AttnShape:
    name: str
    T: int               # tokens (sequences x seq_len)
    seq_len: int
    H: int               # query heads
    Hkv: int             # key/value heads
    dh: int = 128
    base: float = 10000.0
    seed: int = 0

    @property
    def n_seq(self) -> int:
        return self.T // self.seq_len


ATTN_7B = AttnShape("LLaMA-2-7B attention (4 x 4096 tokens, 32 heads of 128)", T=16384,
                    seq_len=4096, H=32, Hkv=32)
ATTN_7B_GQA = AttnShape("grouped-query attention (4 x 4096 tokens, 32 query / 8 kv heads)",
                        T=16384, seq_len=4096, H=32, Hkv=8)


def make_attn_inputs(s: AttnShape, seed: int | None = None) -> dict[str, np.ndarray]:
    """Seeded Q [T, H dh], K and V [T, Hkv dh], dO [T, H dh] as bf16-exact
    float32 arrays."""
    rng = np.random.default_rng(s.seed if seed is None else seed)
    out = {}
    for name, heads in (("Q", s.H), ("K", s.Hkv), ("V", s.Hkv), ("dO", s.H)):
        out[name] = round_to_bf16(rng.standard_normal((s.T, heads * s.dh), dtype=np.float32))
    return out
