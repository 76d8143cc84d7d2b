"""Host logic of the measured-traffic record (no GPU): counter CSVs in the
rocprofv3 layout are reduced to calibrated bytes per launch."""
from __future__ import annotations

import csv

import pytest

from gemm_online_rmsnorm_amd import traffic

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, kib) in enumerate(rows):
            w.writerow({k: 0 for k in FIELDS} | {"Dispatch_Id": i, "Kernel_Name": name,
                                                   "Grid_Size": grid, "Counter_Name": counter,
                                                   "Counter_Value": kib})


def test_calibrated_bytes(tmp_path):
    copy = 1 << 30
    k = "void lr::gemm2_kernel<X>(lr::GemmArgs)"
    # The copy reads 1.25x and writes 0.8x its true size on these counters.
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(traffic.COPY_KERNEL, 64, copy / 1024 * 1.25),
                                            (traffic.COPY_KERNEL, 64, 1.0),
                                            (k, 512, 1000.0), (k, 512, 1200.0), (k, 512, 1100.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(traffic.COPY_KERNEL, 64, copy / 1024 * 0.8),
                                            (k, 512, 400.0), (k, 512, 400.0)])
    rec = traffic.measure(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "gemm2_kernel<X>", copy)
    assert rec["fetch_bytes"] == round(1100.0 * 1024 / 1.25)
    assert rec["write_bytes"] == round(400.0 * 1024 / 0.8)
    assert rec["traffic_bytes"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["dispatches"] == [3, 2] and rec["grid_size"] == 512
    assert rec["source_sha256"] == traffic.source_hash()


def test_mixed_launch_shapes_are_refused(tmp_path):
    k = "void lr::gemm2_kernel<X>(lr::GemmArgs)"
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(traffic.COPY_KERNEL, 64, 10.0), (k, 512, 1.0),
                                            (k, 256, 1.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(traffic.COPY_KERNEL, 64, 10.0), (k, 512, 1.0)])
    with pytest.raises(SystemExit):
        traffic.measure(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "gemm2_kernel<X>", 1024)


def test_stale_record_is_ignored(tmp_path):
    import json
    p = tmp_path / "t.json"
    p.write_text(json.dumps({"source_sha256": "0" * 64, "traffic_bytes": 1}))
    assert traffic.load(str(p)) is None
    p.write_text(json.dumps({"source_sha256": traffic.source_hash(), "traffic_bytes": 1}))
    assert traffic.load(str(p))["traffic_bytes"] == 1


def test_record_follows_its_own_sources(tmp_path):
    """A record names the sources it was taken on; it is valid while they are
    unchanged, whichever kernel family it covers."""
    import json
    k = "attn_dkdv_kernel"
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(traffic.COPY_KERNEL, 64, 512.0), (k, 512, 10.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(traffic.COPY_KERNEL, 64, 1024.0), (k, 512, 5.0)])
    rec = traffic.measure(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), k, 1 << 20,
                          traffic.ATTENTION_SOURCES)
    assert rec["sources"] == list(traffic.ATTENTION_SOURCES)
    assert rec["source_sha256"] == traffic.source_hash(traffic.ATTENTION_SOURCES)
    assert rec["source_sha256"] != traffic.source_hash()
    path = tmp_path / "rec.json"
    path.write_text(json.dumps(rec))
    assert traffic.load(str(path)) == rec
    path.write_text(json.dumps(rec | {"source_sha256": "0" * 64}))
    assert traffic.load(str(path)) is None


def test_bench_reports_a_record_for_its_own_workload_only(tmp_path, monkeypatch):
    """bench.py takes a record for the launch it names and the workload it was
    measured on; the same launch of another workload reports none."""
    import json
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    rec = {"source_sha256": traffic.source_hash(), "sources": list(traffic.KERNEL_SOURCES),
           "traffic_bytes": 123, "bench_name": "SwiGLU recompute + backward", "workload": "7B-bf16"}
    (tmp_path / "traffic_x.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    assert bench._traffic_record("SwiGLU recompute + backward", "7B-bf16") == 123
    assert bench._traffic_record("SwiGLU recompute + backward", "1B-bf16") is None
    assert bench._traffic_record("dgu_r", "7B-bf16") is None
