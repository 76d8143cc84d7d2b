"""Shared pieces of the GPU parity tests."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

BF16_TOL = 1e-2   # max|gpu - oracle| / max|oracle|, bf16 storage
F32_TOL = 1e-5    # same metric, fp32 everywhere


def gpu_or_skip():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gemm_online_rmsnorm_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("liblrblock.so is not built: run __graft_entry__.build() first")
    _lib.load()
    return torch


def say(*a):
    """Progress line that reaches the log even under output capture."""
    print(*a, file=sys.stderr, flush=True)


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    return num / (den if den > 0 else 1.0)


class ErrAcc:
    """max|gpu - ref| and max|ref| per tensor, accumulated over row blocks."""

    def __init__(self):
        self.num = {}
        self.den = {}

    def add(self, name, gpu, ref):
        gpu = np.asarray(gpu, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
        if not np.all(np.isfinite(gpu)):
            self.num[name] = float("inf")
        self.num[name] = max(self.num.get(name, 0.0), float(np.max(np.abs(gpu - ref))))
        self.den[name] = max(self.den.get(name, 0.0), float(np.max(np.abs(ref))))

    def errors(self):
        return {k: self.num[k] / (self.den[k] if self.den[k] > 0 else 1.0) for k in self.num}

    def check(self, tol, label=""):
        errs = self.errors()
        worst = max(errs.items(), key=lambda kv: kv[1])
        say(f"[parity {label}] worst {worst[0]} {worst[1]:.3e} (tol {tol:g}); " +
            " ".join(f"{k}={v:.1e}" for k, v in sorted(errs.items())))
        bad = {k: v for k, v in errs.items() if not (v <= tol)}
        assert not bad, f"{label}: over tolerance {tol}: {bad}"
        return errs
