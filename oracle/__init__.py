"""fp64 CPU oracle of the low-rank decoder-block linear stack (BOOST).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only the tests, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it. It
shares no code with the GPU library and imports nothing from it.

It is a plain, slow, float64 implementation written from the BOOST pages:
  * the project page (alvin-zyl.github.io/boost), sections "Move the chunk
    boundary to the bottleneck" (the factorised block, the chunk shift, the
    all-reduce volume table) and "Three supporting changes" (Online RMSNorm,
    linear layer grouping, checkpointing without communication);
  * the awesome-system-papers summary (BOOST-MLSys26), section "核心方法"
    (the correction factor alpha = RMS_local / RMS_global applied per row,
    and the batched GEMM over (input, weight) pairs).

Every fast form of the method reaches the plain result exactly (up to
rounding order), so the oracle is the plain block written out, plus each fast
form computed on its own so that tests can check them against it.

Parity status of each function is stated in its docstring; the pins live in
``tests/test_oracle_*.py``.
"""
from .block import (  # noqa: F401
    silu,
    silu_grad,
    rms,
    rmsnorm,
    online_rmsnorm_matmul,
    block_forward,
    block_forward_online,
    block_forward_grouped,
    block_backward,
    block_backward_tape,
    block_loss,
    GRAD_NAMES,
)
from .share import (  # noqa: F401
    shard_weights,
    share_forward,
    share_backward,
    simulate_tp_forward,
    simulate_tp_backward,
)
from .blocked import run_fwd_bwd, grouped_views  # noqa: F401
