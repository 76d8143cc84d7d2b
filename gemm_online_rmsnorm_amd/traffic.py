"""Measured HBM traffic of one kernel from rocprofv3 counter runs.

Two counter runs of the same command, one collecting FETCH_SIZE and one
WRITE_SIZE (KiB per dispatch, read from the L2 channels), are turned into
bytes per launch of one kernel. The counters are calibrated against a plain
device copy of known size made in the same process (bench.py
--copy-calibration): the scale factor of each counter is the copy's true
byte count over what the counter read for it.

    rocprofv3 --pmc FETCH_SIZE -d D1 -o f -f csv -- python bench.py --copy-calibration ...
    rocprofv3 --pmc WRITE_SIZE -d D2 -o w -f csv -- python bench.py --copy-calibration ...
    python -m gemm_online_rmsnorm_amd.traffic D1/.../f_counter_collection.csv \\
        D2/.../w_counter_collection.csv --bench-name "SwiGLU recompute + backward" \\
        --kernel "gemm2_kernel<...>" --workload 7B-bf16 --copy-bytes N -o profiles/<name>.json

The result carries a hash of the kernel sources and the name of the workload
it was measured on; bench.py reports it only for that workload and while the
sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


# Sources of the block's GEMM and memory-bound kernels and their launch
# code (the attention kernels and the C ABI layer are built from other files).
KERNEL_SOURCES = ("lr_kernels.hip", "lr_common.hpp", "lr_gemm.hpp", "lr_gemm2.hpp",
                  "lr_internal.hpp")
# Sources of the attention kernels and their launch code.
ATTENTION_SOURCES = ("lr_attention.hip", "lr_attn.hpp")


def source_hash(sources=KERNEL_SOURCES) -> str:
    """SHA-256 over the named kernel sources (files of csrc/)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name in sources:
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _per_dispatch(path: str, counter: str) -> dict[str, list[tuple[int, float]]]:
    """kernel name -> [(grid size, counter value in KiB)] per dispatch."""
    out: dict[str, list[tuple[int, float]]] = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(
                (int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def _match(table: dict, needle: str) -> list[tuple[int, float]]:
    hits = [k for k in table if needle in k]
    if len(hits) != 1:
        raise SystemExit(f"kernel filter {needle!r} matches {len(hits)} kernels: {hits[:4]}")
    return table[hits[0]]


def measure(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int,
            sources=KERNEL_SOURCES) -> dict:
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    kf, kw = _match(fetch, kernel), _match(write, kernel)
    grids = {g for g, _ in kf} | {g for g, _ in kw}
    if len(grids) != 1:
        raise SystemExit(f"{kernel!r} ran with several grid sizes {sorted(grids)}; "
                         "its launches are not one workload")
    # The copy: the largest dispatch of the blit kernel is the calibration copy.
    cf = max(v for _, v in _match(fetch, COPY_KERNEL))
    cw = max(v for _, v in _match(write, COPY_KERNEL))
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    fetch_b = statistics.median(v for _, v in kf) * 1024.0 * f_scale
    write_b = statistics.median(v for _, v in kw) * 1024.0 * w_scale
    return {
        "kernel": kernel, "dispatches": [len(kf), len(kw)], "grid_size": grids.pop(),
        "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
        "traffic_bytes": round(fetch_b + write_b),
        "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "sources": list(sources), "source_sha256": source_hash(sources),
    }


def load(path: str) -> dict | None:
    """The stored measurement if it was taken on the current sources, else None."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    sources = tuple(rec.get("sources", KERNEL_SOURCES))
    return rec if rec.get("source_sha256") == source_hash(sources) else None


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--kernel", required=True, help="substring of the kernel's name")
    ap.add_argument("--bench-name", required=True, help="the launch's name in bench.py")
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--workload", required=True,
                    help="the profiled workload's name (bench.py reports the record for it only)")
    ap.add_argument("--command", default="", help="the profiled command, for the record")
    ap.add_argument("--attention", action="store_true",
                    help="an attention kernel: hash the attention sources")
    ap.add_argument("-o", "--out", required=True)
    a = ap.parse_args()
    rec = measure(a.fetch_csv, a.write_csv, a.kernel, a.copy_bytes,
                  ATTENTION_SOURCES if a.attention else KERNEL_SOURCES)
    rec["bench_name"] = a.bench_name
    rec["workload"] = a.workload
    rec["command"] = a.command
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
