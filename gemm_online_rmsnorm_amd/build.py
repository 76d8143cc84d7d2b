"""Build liblrblock.so for gfx950 in-tree with hipcc.

    python -m gemm_online_rmsnorm_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblrblock.so")
SOURCES = ("lr_kernels.hip", "lr_attention.hip", "lr_api.cpp")
ARCH = os.environ.get("LRBLOCK_ARCH", "gfx950")
# The attention backward keeps its dK/dV accumulators and K/V fragments in
# registers past 256 VGPRs; the VGPR form of the MFMA instructions lets the
# compiler hold them without copying through AGPRs on every iteration.
EXTRA = {"lr_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise FileNotFoundError("hipcc not found")


def flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="lrblock_build_") as tmp:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [hipcc, *flags(), *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src),
                   "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                            if "packed-fp32-ops" not in l)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
            return obj

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_out = OUT + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
        os.replace(tmp_out, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
