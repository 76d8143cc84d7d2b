"""Device buffers for one block workload and calls of the C ABI on them.

Plumbing for tests, the benchmark and the smoke check: it uploads host
arrays (the seeded inputs) as torch device tensors in the block's storage
type, stacks the grouped down-projection weights, allocates the outputs,
saved activations, gradients and workspaces once, and runs lr_block_fwd /
lr_block_bwd on them. Every arithmetic step runs in the library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (LR_BF16, LR_F32, LR_STAGE_ALL, alloc_workspace, block_bwd, block_fwd,
               block_shape, torch_dtype)

GRAD_KEYS = {  # gradient tensor name in the results -> weight field
    "dgamma1": "gamma1", "dgamma2": "gamma2", "dA_qkv": "A_qkv", "dB_q": "B_q",
    "dB_k": "B_k", "dB_v": "B_v", "dA_o": "A_o", "dB_o": "B_o", "dA_gu": "A_gu",
    "dB_g": "B_g", "dB_u": "B_u", "dA_dn": "A_dn", "dB_dn": "B_dn",
}


class BlockRun:
    """All device state of one block workload.

    inputs: host float32 arrays keyed X, O, gamma1, gamma2, A_q, A_k, A_v,
    B_q, B_k, B_v, A_o, B_o, A_g, A_u, B_g, B_u, A_dn, B_dn, dY, dQ, dK, dV.
    """

    def __init__(self, T, d, r, F, D, P, dtype: str, eps: float, partials: bool, inputs,
                 device="cuda", heads=1):
        self.dt = LR_BF16 if dtype == "bf16" else LR_F32
        self.tdt = torch_dtype(self.dt)
        self.shape = block_shape(T, d, r, F, d_norm=D, n_panels=P, n_heads=heads, eps=eps,
                                 dtype=self.dt, emit_partials=partials)
        self.T, self.d, self.r, self.F, self.P = T, d, r, F, P
        self.partials = partials
        dev = torch.device(device)
        self.device = dev

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(self.tdt)

        self.X, self.O = up(inputs["X"]), up(inputs["O"])
        self.dY, self.dQ = up(inputs["dY"]), up(inputs["dQ"])
        self.dK, self.dV = up(inputs["dK"]), up(inputs["dV"])
        self.W = {
            "gamma1": up(inputs["gamma1"]), "gamma2": up(inputs["gamma2"]),
            "A_qkv": up(np.concatenate([inputs["A_q"], inputs["A_k"], inputs["A_v"]], 0)),
            "B_q": up(inputs["B_q"]), "B_k": up(inputs["B_k"]), "B_v": up(inputs["B_v"]),
            "A_o": up(inputs["A_o"]), "B_o": up(inputs["B_o"]),
            "A_gu": up(np.concatenate([inputs["A_g"], inputs["A_u"]], 0)),
            "B_g": up(inputs["B_g"]), "B_u": up(inputs["B_u"]),
            "A_dn": up(inputs["A_dn"]), "B_dn": up(inputs["B_dn"]),
        }

        def empty(*s, dt=None):
            return torch.empty(*s, dtype=dt or self.tdt, device=dev)

        self.out = {k: empty(T, d) for k in ("Q", "K", "V", "Y")}
        self.saved = {"qkv_r": empty(T, 3 * r), "o_r": empty(T, r), "gu_r": empty(T, 2 * r),
                      "d_r": empty(T, r), "rms1": empty(T, dt=torch.float32),
                      "rms2": empty(T, dt=torch.float32)}
        self.part = None
        if partials:
            self.part = {"P_qkv": empty(T, 3 * r), "P_gu": empty(T, 2 * r),
                         "ss1": empty(T, dt=torch.float32), "ss2": empty(T, dt=torch.float32)}
        elif P > 1:
            self.part = {"ss1": empty(P, T, dt=torch.float32),
                         "ss2": empty(P, T, dt=torch.float32)}
        self.dX, self.dO = empty(T, d), empty(T, d)
        self.grads = {f: torch.empty_like(self.W[f], dtype=torch.float32) for f in self.W}
        self.ws_f = alloc_workspace(self.shape, False, dev)
        self.ws_b = alloc_workspace(self.shape, True, dev)

    def fwd(self, stage=LR_STAGE_ALL, stream=None):
        block_fwd(self.shape, self.W, self.X, self.O, self.out, self.saved, self.part, stage,
                  self.ws_f, stream)

    def bwd(self, stage=LR_STAGE_ALL, stream=None):
        block_bwd(self.shape, self.W, self.X, self.O, self.saved, self.dY, self.dQ, self.dK,
                  self.dV, self.dX, self.dO, self.grads, stage, self.ws_b, stream)

    def step(self, stream=None):
        self.fwd(stream=stream)
        self.bwd(stream=stream)

    def results(self, host_dtype=np.float64) -> dict:
        """Download every output (names as in oracle.run_fwd_bwd)."""
        torch.cuda.synchronize(self.device)

        def h(t):
            return t.float().cpu().numpy().astype(host_dtype, copy=False)

        res = {k: h(v) for k, v in self.out.items()}
        res.update({k: h(v) for k, v in self.saved.items()})
        if self.part is not None:
            if self.partials:
                res.update({k: h(v) for k, v in self.part.items()})
            else:
                res["ss_panels1"] = h(self.part["ss1"])
                res["ss_panels2"] = h(self.part["ss2"])
        res["dX"], res["dO"] = h(self.dX), h(self.dO)
        for k, f in GRAD_KEYS.items():
            res[k] = h(self.grads[f])
        return res
