"""bench.py's command-line contract that holds without a GPU: more than one
GPU is refused with a message and exit status 2, and without a GPU the
benchmark says so instead of falling back to the CPU."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, env=e, timeout=600)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and "not supported" in r.stderr
    assert r.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    r = _run(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE=4" in r.stderr


def test_no_gpu_no_fallback():
    import torch
    if torch.cuda.is_available():
        return  # covered by the GPU runs
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_parity_field_of_the_bench_line():
    """bench.parity: the worst tensor over every output, the weight gradients
    only when the oracle ran every row, and a non-finite value as a failure."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    rng = np.random.default_rng(0)
    ref = {"Y": rng.standard_normal((8, 4)), "dX": rng.standard_normal((8, 4)),
           "dA_qkv": rng.standard_normal((3, 4)), "ss_panels1": rng.random((2, 8))}
    gpu = {k: v.astype(np.float32) for k, v in ref.items()}
    gpu["Y"] = gpu["Y"] + np.float32(0.05) * np.max(np.abs(ref["Y"]))
    p = bench.parity(gpu, ref, 8, 8, 1e-2)
    assert p["n_tensors"] == 4 and p["tensor"] == "Y" and not p["ok"]
    assert abs(p["worst"] - 0.05) < 1e-6
    # only 5 rows: no weight gradient; rows past 5 are not compared
    gpu["Y"] = ref["Y"].astype(np.float32)
    gpu["dX"][6:] = np.nan
    p = bench.parity(gpu, {k: (v[:, :5] if k == "ss_panels1" else
                               (v if k == "dA_qkv" else v[:5])) for k, v in ref.items()}, 5, 8,
                     1e-2)
    assert p["n_tensors"] == 3 and p["ok"] and p["worst"] < 1e-6
    gpu["Y"][0, 0] = np.inf
    assert not bench.parity(gpu, ref, 8, 8, 1e-2)["ok"]
