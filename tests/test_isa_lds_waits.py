"""Static check of the GEMM engine's machine code: transposing LDS reads.

The pipelined engine issues ds_read_b64_tr_b16 through inline assembly, so
the compiler does not track when their results land; the kernel waits for
them itself (s_waitcnt lgkmcnt(0)) before any use. This test compiles the
kernels for gfx950 and runs a data-flow pass over every kernel's control
flow graph: no instruction may touch a register written by such a read
before an lgkmcnt(0) wait on every path between them. CPU only (hipcc
cross-compiles).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from gemm_online_rmsnorm_amd import build as lrbuild

REG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\S+)")


def _regs(text: str) -> set[int]:
    out: set[int] = set()
    for m in REG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _blocks(lines: list[str]):
    """Basic blocks of one function: (label, instructions, successors)."""
    blocks, cur, label = [], [], "entry"
    for ln in lines:
        t = ln.split(";")[0].strip()
        if not t or t.startswith("."):
            if t.startswith(".LBB") and t.endswith(":"):
                blocks.append([label, cur, None])
                label, cur = t[:-1], []
            continue
        cur.append(t)
        if BRANCH.match(t) or t.startswith("s_endpgm"):
            blocks.append([label, cur, None])
            label, cur = f"{label}+", []
    blocks.append([label, cur, None])
    names = [b[0] for b in blocks]
    for i, b in enumerate(blocks):
        succ = []
        last = b[1][-1] if b[1] else ""
        m = BRANCH.match(last)
        if last.startswith("s_endpgm"):
            pass
        elif m and m.group(1) == "branch":
            succ.append(m.group(2))
        else:
            if m:
                succ.append(m.group(2))
            if i + 1 < len(blocks):
                succ.append(names[i + 1])
        b[2] = [s for s in succ if s in names]
    return blocks


def _check_function(name: str, lines: list[str]) -> list[str]:
    blocks = _blocks(lines)
    index = {b[0]: i for i, b in enumerate(blocks)}
    state_in = [set() for _ in blocks]
    errors: list[str] = []
    changed = True
    while changed:
        changed = False
        for i, (label, insts, succ) in enumerate(blocks):
            pend = set(state_in[i])
            for t in insts:
                op = t.split()[0]
                if op == "s_waitcnt":
                    if "lgkmcnt(0)" in t:
                        pend.clear()
                    continue
                regs = _regs(t)
                hit = regs & pend
                if hit:
                    msg = f"{name} {label}: '{t}' uses pending v{sorted(hit)[0]}"
                    if msg not in errors:
                        errors.append(msg)
                if op == "ds_read_b64_tr_b16":
                    dst = t.split(None, 1)[1].split(",")[0]
                    pend |= _regs(dst)
            for s in succ:
                j = index[s]
                if not pend <= state_in[j]:
                    state_in[j] |= pend
                    changed = True
    return errors


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "lr_kernels.s"
    cmd = [hipcc, *lrbuild.flags(), "--cuda-device-only", "-S",
           os.path.join(lrbuild.CSRC, "lr_kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _functions(asm: str):
    for m in re.finditer(r"^(_Z\S+):\s*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        yield name, asm[m.end():end].splitlines()


def test_transposed_reads_are_waited_for(kernel_asm):
    n_checked, errors = 0, []
    for name, lines in _functions(kernel_asm):
        if not any("ds_read_b64_tr_b16" in l for l in lines):
            continue
        n_checked += 1
        errors += _check_function(name, lines)
    assert n_checked > 0, "no kernel uses transposing LDS reads"
    assert not errors, "\n".join(errors[:20])


def test_checker_flags_a_missing_wait():
    """The data-flow pass itself: a use before the wait is reported, a use
    after it is not, and a pending read survives a loop back edge."""
    bad = ["ds_read_b64_tr_b16 v[4:5], v1", "v_mov_b32_e32 v9, v5", "s_endpgm"]
    good = ["ds_read_b64_tr_b16 v[4:5], v1", "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v9, v5",
            "s_endpgm"]
    loop = [".LBB0_1:", "v_mov_b32_e32 v9, v5", "ds_read_b64_tr_b16 v[4:5], v1",
            "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert _check_function("bad", bad)
    assert not _check_function("good", good)
    assert _check_function("loop", loop)
