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
