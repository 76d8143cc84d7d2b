#!/usr/bin/env python3
"""Benchmark of the low-rank decoder-block linear stack on one MI355X.

One step = the block's forward and backward (lr_block_fwd + lr_block_bwd)
over one batch of 16384 synthetic tokens, with every input already resident
in HBM. Prints ONE JSON line:
  value          tokens/s of fwd+bwd (T / step time)
  tflops         algorithmic TFLOP/s including the mandated recompute
  roofline       the dominant kernel against the bf16 MFMA peak, from HIP
                 events recorded around its launches on its stream
  hbm_phases     every memory-bound kernel (row dots, gamma folds, split-K
                 sums, column sums, rank-share finalize): GPU-side time per
                 launch (20 launches back to back between two events),
                 algorithmic bytes, GB/s and fraction of HBM bandwidth
  cpu_baseline   the fp64 CPU oracle on a bounded sample of the same
                 workload (all 16384 tokens by default), on this host's cores
  parity         the outputs of the timed configuration against that oracle
                 run: max|gpu - oracle| / max|oracle| over every output,
                 saved activation and gradient; the exit status is 3 when
                 it exceeds 1e-2 (bf16) or 1e-5 (fp32)

    python bench.py [--steps 8] [--warmup 2] [--config 3]

The default workload is the 7B-shape block (d = 4096, r = 1024,
d_ff = 11008); the other workloads are parity-test cases.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3    # MI355X dense fp32
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
COPY_BYTES = 1 << 30             # calibration copy for the byte counters
HBM_REPEAT = 20                  # back-to-back launches per memory-bound measurement
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3: 7B shape)")
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="tokens of the workload the CPU oracle runs for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels", action="store_true", help="also print the per-kernel table")
    ap.add_argument("--tp-split", type=int, default=0, metavar="k",
                    help="instead of the block step: time one rank's GEMMs of the config's "
                         "block under the vanilla and the bottleneck-aware split over k ranks")
    ap.add_argument("--attention", choices=("mha", "gqa", "block"), default=None,
                    help="instead of the block step: causal RoPE attention fwd+bwd at the "
                         "LLaMA-2-7B attention shape (mha: 32 kv heads, gqa: 8), or "
                         "(block) the whole decoder block: the config's linear stack with "
                         "attention between its stages")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step into a HIP graph and time K replays of it "
                         "instead of K eager steps")
    ap.add_argument("--vendor-gemms", action="store_true",
                    help="instead of the block step: time torch.matmul (hipBLASLt) on plain "
                         "GEMMs of the config's shapes, a reference point for the library's "
                         "fused kernels (no fusion, random operands)")
    ap.add_argument("--gemm-sweep", action="store_true",
                    help="instead of the block step: time one-pair products of the block's "
                         "widths (16384 x 4096, NT, NT with a residual, NN; 4096 x 4096 TN) at "
                         "K = 1024 ... 8192 through the C ABI and fit time = a + b K, the "
                         "per-launch fixed cost and the main-loop rate")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"first make one device copy of {COPY_BYTES} bytes, the reference "
                         "rocprofv3 byte counters are scaled by")
    return ap.parse_args()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(s, inputs, rows):
    """The oracle as it stands, timed on a bounded sample of the workload.
    Returns the cpu_baseline record and the oracle's outputs (for parity)."""
    import numpy as np
    import oracle
    threads = _blas_threads()
    rows = min(rows, s.T)
    sample = {k: (v[:rows] if v.shape[0] == s.T and k in ("X", "O", "dY", "dQ", "dK", "dV")
                  else v) for k, v in inputs.items()}
    t0 = time.perf_counter()
    out = oracle.run_fwd_bwd(sample, D=s.D, eps=s.eps, n_panels=s.P, partials=s.partials,
                             row_block=2048)
    dt = time.perf_counter() - t0
    assert np.isfinite(out["dA_qkv"]).all()
    rec = {"value": rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "seconds": round(dt, 2), "cpu_model": _cpu_model(),
           "host_cpus": len(os.sched_getaffinity(0)),
           "sample": f"first {rows} of {s.T} tokens of the {s.name} workload, full fwd+bwd "
                     f"incl. weight grads, numpy float64 (OpenBLAS, {threads} threads)"}
    return rec, out, rows


def parity(gpu, ref, rows, T, tol):
    """max|gpu - oracle| / max|oracle| per tensor on the oracle's rows (every
    tensor, weight gradients included, when it ran all T rows)."""
    import numpy as np
    worst_k, worst, errs = None, 0.0, {}
    for k, v in ref.items():
        g = gpu[k]
        if rows < T:
            if k.startswith("d") and k not in ("dX", "dO"):
                continue  # weight and gamma gradients need every row
            g = g[:, :rows] if k.startswith("ss_panels") else g[:rows]
        den = float(np.max(np.abs(v))) or 1.0
        e = float(np.max(np.abs(np.asarray(g, dtype=np.float64) - v))) / den
        if not np.all(np.isfinite(g)):
            e = float("inf")
        errs[k] = e
        if not e <= worst:
            worst_k, worst = k, e
    return {"worst": worst, "tensor": worst_k, "tol": tol, "n_tensors": len(errs),
            "rows": rows, "ok": bool(worst <= tol),
            "metric": "max|gpu - oracle| / max|oracle| per tensor, fp64 oracle"}


def tp_split_main(args, s):
    """One JSON line: one rank's GEMM time, TFLOP/s and arithmetic intensity
    under the vanilla and the bottleneck-aware split of the config's block
    over k ranks (same kernels, synthetic operands), and the all-reduce
    values per token each split sends."""
    from gemm_online_rmsnorm_amd import tp_split as tps
    k = args.tp_split
    if s.dtype != "bf16" or s.partials or s.d % k or s.r % k or s.F % k:
        print(f"--tp-split needs a bf16 full-block config whose d, r, d_ff split {k} ways",
              file=sys.stderr)
        sys.exit(2)
    print(f"[bench] tp split k={k} of {s.name}", file=sys.stderr, flush=True)
    out = {"metric": f"one rank's block GEMMs under tensor parallelism over {k} GPUs",
           "unit": "ms", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": f"{s.name} block, rank 0 of {k}",
                                           "tokens": s.T, "d": s.d, "r": s.r, "d_ff": s.F}}
    for split, fn in (("vanilla", tps.vanilla_gemms), ("bottleneck", tps.btp_gemms)):
        rows = tps.time_split(fn(s.T, s.d, s.r, s.F, k))
        summ = tps.summarize(rows, MFMA_BF16_PEAK_TFLOPS)
        summ["allreduce_values_per_token"] = tps.allreduce_values_per_token(
            "vanilla" if split == "vanilla" else "btp", s.d, s.r, s.F)
        summ["gemms"] = [{k2: v for k2, v in r.items() if k2 not in ("flops", "bytes")}
                         for r in rows]
        out[split] = summ
    out["value"] = out["bottleneck"]["ms"]
    out["mlp_intensity_ratio"] = round(out["bottleneck"]["mlp"]["flop_per_byte"]
                                       / out["vanilla"]["mlp"]["flop_per_byte"], 2)
    out["speedup"] = round(out["vanilla"]["ms"] / out["bottleneck"]["ms"], 3)
    print(json.dumps(out))


def _graph(torch, step):
    """Capture step(None) (every library call on the current stream) into a
    HIP graph, after one eager call on the capture's side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(None)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(None)
    torch.cuda.synchronize()
    return g


def _timed_step(torch, args, step, stream):
    """What one timed step runs: an eager step on `stream`, or with --graph a
    replay (on the current stream, which is `stream`) of its captured graph."""
    if not args.graph:
        return lambda: step(stream)
    g = _graph(torch, step)
    return g.replay


def _calibration_copy(torch):
    """One device copy of COPY_BYTES: the reference rocprofv3's byte counters
    are scaled by (gemm_online_rmsnorm_amd/traffic.py)."""
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def _traffic_record(bench_name, workload):
    """Measured HBM bytes per launch of the named launch, from the record in
    profiles/ taken on the current kernel sources and on this workload; None
    without one."""
    from gemm_online_rmsnorm_amd import traffic as lrtraffic
    if not os.path.isdir(TRAFFIC_DIR):
        return None
    for name in sorted(os.listdir(TRAFFIC_DIR)):
        if name.startswith("traffic_") and name.endswith(".json"):
            rec = lrtraffic.load(os.path.join(TRAFFIC_DIR, name))
            if rec and rec.get("bench_name") == bench_name and rec.get("workload") == workload:
                return rec["traffic_bytes"]
    return None


def vendor_gemms_main(args, s):
    """One JSON line: torch.matmul (hipBLASLt on ROCm) on plain bf16 GEMMs
    with the shapes of the block's products, each timed over K calls after
    W warm-up calls. Nothing here is part of the library's path."""
    import torch

    T, d, r, F = s.T, s.d, s.r, s.F
    shapes = [  # name, M, N, K, operand layout
        ("QKV down-projection (3r x d)", T, 3 * r, d, "NT"),
        ("one up-projection (d x r)", T, d, r, "NT"),
        ("one gate/up up-projection (d_ff x r)", T, F, r, "NT"),
        ("down-projection (r x d_ff)", T, r, F, "NT"),
        ("weight gradient dB_g (d_ff x r over T)", F, r, T, "TN"),
        ("weight gradient dB_dn (d x r over T)", d, r, T, "TN"),
    ]
    g = torch.Generator(device="cuda").manual_seed(0)
    out = []
    for name, M, N, K, lay in shapes:
        if lay == "NT":
            a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
            b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16, generator=g)
            fn = lambda a=a, b=b: a @ b.t()
        else:
            a = torch.randn(K, M, device="cuda", dtype=torch.bfloat16, generator=g)
            b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16, generator=g)
            fn = lambda a=a, b=b: a.t() @ b
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        out.append({"gemm": name, "M": M, "N": N, "K": K, "layout": lay, "ms": round(ms, 4),
                    "tflops": round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)})
        del a, b
    print(json.dumps({"metric": "torch.matmul (hipBLASLt) bf16 TFLOP/s on the block's GEMM "
                                "shapes (reference point)", "n_gpus": 1,
                      "config": {"workload": s.name, "tokens": T, "d": d, "r": r, "d_ff": F},
                      "gemms": out}), flush=True)


def gemm_sweep_main(args):
    """One JSON line: per-launch time of single products through
    lr_grouped_lowrank_gemm at K = 1024, 2048, 4096, 8192 (M = 16384,
    N = 4096; the weight gradient 4096 x 4096 over K), and the least-squares
    fit time = a + b * K per product: a is the per-launch cost that does not
    grow with K (prologue, epilogue, launch), b the main loop's time per k."""
    import ctypes
    import torch
    from gemm_online_rmsnorm_amd import _lib

    lib = _lib.load()
    P = _lib.lr_gemm_pair
    g = torch.Generator(device="cuda").manual_seed(0)
    M, N, KMAX = 16384, 4096, 8192

    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, device="cuda", generator=g) * scale).to(torch.bfloat16)

    X, Wt, Wn = rnd(M, KMAX), rnd(N, KMAX, scale=0.01), rnd(KMAX, N, scale=0.01)
    Y, R = torch.empty(M, N, device="cuda", dtype=torch.bfloat16), rnd(M, N)
    A, B = rnd(KMAX, N), rnd(KMAX, N)
    C = torch.empty(N, N, device="cuda", dtype=torch.float32)
    ws = torch.empty(64 << 20, device="cuda", dtype=torch.uint8)
    st = torch.cuda.current_stream().cuda_stream
    x, wt, wn, y, r = X.data_ptr(), Wt.data_ptr(), Wn.data_ptr(), Y.data_ptr(), R.data_ptr()
    ks = (1024, 2048, 4096, 8192)
    prods = {
        "NT": lambda K: (P(M, N, K, x, KMAX, wt, KMAX, y, N, None, 0), 0, 0, 2.0 * M * N * K),
        "NT + residual": lambda K: (P(M, N, K, x, KMAX, wt, KMAX, y, N, r, N), 0, 1,
                                    2.0 * M * N * K),
        "NN": lambda K: (P(M, N, K, x, KMAX, wn, N, y, N, None, 0), 1, 0, 2.0 * M * N * K),
        "TN (weight gradient)": lambda K: (P(N, N, K, A.data_ptr(), N, B.data_ptr(), N,
                                             C.data_ptr(), N, None, 0), 2, 0, 2.0 * N * N * K),
    }
    # Every (product, K) point once per round, in turn, over three rounds; a
    # point keeps its fastest round (the clock moves with the power draw).
    best = {}
    for _ in range(3):
        for name, mk in prods.items():
            for K in ks:
                pair, layout, epi, flop = mk(K)
                arr = (P * 1)(pair)
                nbytes = int(lib.lr_grouped_lowrank_gemm_workspace_bytes(1, arr, _lib.LR_BF16,
                                                                         layout))
                assert nbytes <= ws.numel()

                def call():
                    _lib.check(lib.lr_grouped_lowrank_gemm_ws(
                        1, arr, _lib.LR_BF16, layout, epi, ctypes.c_void_p(ws.data_ptr()),
                        ws.numel(), st))
                for _ in range(max(1, args.warmup)):
                    call()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(args.steps):
                    call()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / args.steps * 1e3
                best[name, K] = min(best.get((name, K), us), us)
    out = []
    for name, mk in prods.items():
        pts = [{"K": K, "us": round(best[name, K], 1),
                "tflops": round(mk(K)[3] / best[name, K] / 1e6, 1)} for K in ks]
        n = len(ks)
        mk_, mt = sum(ks) / n, sum(p["us"] for p in pts) / n
        b = (sum((k - mk_) * (p["us"] - mt) for k, p in zip(ks, pts))
             / sum((k - mk_) ** 2 for k in ks))
        a = mt - b * mk_
        flop_per_k = mk(1)[3]
        out.append({"product": name, "points": pts, "fixed_us": round(a, 1),
                    "us_per_1024_k": round(b * 1024, 2),
                    "main_loop_tflops": round(flop_per_k / (b * 1e-6) / 1e12, 1)})
    print(json.dumps({"metric": "one-pair product time vs K (C ABI, bf16)", "n_gpus": 1,
                      "steps": args.steps, "config": {"M": M, "N": N, "tn_out": [N, N]},
                      "products": out}), flush=True)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def block_attention_main(args):
    """One JSON line: the whole decoder block, forward + backward: the
    low-rank linear stack of the config (7B by default) split at the
    attention core, with causal RoPE attention (4 sequences of 4096 tokens,
    heads of 128) between the stages, as a trainer chains the entry points."""
    import torch

    import synth
    import gemm_online_rmsnorm_amd as lr
    from gemm_online_rmsnorm_amd.runner import BlockRun

    s = synth.config(args.config)
    if s.dtype != "bf16" or s.partials or s.d % 128 or s.T % 4096:
        print("--attention block needs a bf16 full-block config with d a multiple of 128",
              file=sys.stderr)
        sys.exit(2)
    heads, seq_len = s.d // 128, 4096
    print(f"[bench] decoder block {s.name} with attention ({heads} heads of 128)",
          file=sys.stderr, flush=True)
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials, synth.make_inputs(s),
                   heads=heads)
    ashape = lr.attn_shape(s.T, seq_len, heads, heads, 128)
    lse = torch.empty(heads, s.T, dtype=torch.float32, device="cuda")
    wsf = torch.empty(lr.attention_workspace_bytes(ashape, False), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(lr.attention_workspace_bytes(ashape, True), dtype=torch.uint8,
                      device="cuda")
    stream = torch.cuda.current_stream()
    Q, K, V = run.out["Q"], run.out["K"], run.out["V"]

    def step(st):
        run.fwd(stage=lr.LR_STAGE_PRE_ATTN, stream=st)
        lr.attention_fwd(ashape, Q, K, V, run.O, lse, ws=wsf, stream=st)
        run.fwd(stage=lr.LR_STAGE_POST_ATTN, stream=st)
        run.bwd(stage=lr.LR_STAGE_POST_ATTN, stream=st)
        lr.attention_bwd(ashape, Q, K, V, run.O, run.dO, lse, run.dQ, run.dK, run.dV, ws=wsb,
                         stream=st)
        run.bwd(stage=lr.LR_STAGE_PRE_ATTN, stream=st)

    for _ in range(args.warmup):
        step(stream)
    timed = _timed_step(torch, args, step, stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        timed()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    pairs = (s.T // seq_len) * seq_len * (seq_len + 1) / 2
    flop = s.T * (s.fwd_flop_per_token() + s.bwd_flop_per_token()
                  + s.recompute_flop_per_token()) + 14 * 128 * pairs * heads
    tflops = flop / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "whole decoder block (low-rank linear stack + causal RoPE attention) "
                  "fwd+bwd tokens/s",
        "value": round(s.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "launch": "hip graph" if args.graph else "eager",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs and random-init factors)",
        "config": {"workload": f"{s.name} block with attention", "tokens": s.T,
                   "seq_len": seq_len, "heads": heads, "d": s.d, "r": s.r, "d_ff": s.F},
        "tflops": round(tflops, 1), "mfma_peak_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
    }), flush=True)


def attention_main(args):
    """One JSON line: causal RoPE attention, forward + backward, at the
    LLaMA-2-7B attention shape (4 sequences of 4096 tokens, 32 query heads
    of 128). TFLOP/s counts the products one pass needs over the unmasked
    (query, key) pairs: 4 * 128 flops per pair and head forward, 10 * 128
    backward; the split backward kernels recompute the scores and dP."""
    import numpy as np
    import torch

    import synth
    import gemm_online_rmsnorm_amd as lr

    s = synth.ATTN_7B_GQA if args.attention == "gqa" else synth.ATTN_7B
    print(f"[bench] attention {s.name}", file=sys.stderr, flush=True)
    inp = synth.make_attn_inputs(s)
    dev = {k: torch.from_numpy(v).cuda().to(torch.bfloat16) for k, v in inp.items()}
    Q, K, V, dO = dev["Q"], dev["K"], dev["V"], dev["dO"]
    shape = lr.attn_shape(s.T, s.seq_len, s.H, s.Hkv, s.dh, s.base)
    O = torch.empty_like(Q)
    lse = torch.empty(s.H, s.T, dtype=torch.float32, device="cuda")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    wsf = torch.empty(lr.attention_workspace_bytes(shape, False), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(lr.attention_workspace_bytes(shape, True), dtype=torch.uint8,
                      device="cuda")
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        _calibration_copy(torch)

    def step(st):
        lr.attention_fwd(shape, Q, K, V, O, lse, ws=wsf, stream=st)
        lr.attention_bwd(shape, Q, K, V, O, dO, lse, dQ, dK, dV, ws=wsb, stream=st)

    for _ in range(args.warmup):
        step(stream)
    timed = _timed_step(torch, args, step, stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        timed()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    lr.profile_enable(True)
    for _ in range(args.steps):
        step(stream)
    torch.cuda.synchronize()
    lr.profile_enable(False)
    prof = lr.profile_collect()

    pairs = s.n_seq * s.seq_len * (s.seq_len + 1) / 2   # unmasked (query, key) pairs
    per_pair = {"attention fwd": 4, "attention bwd dQ": 6, "attention bwd dK dV": 8}
    kernels = []
    for name, count, total in prof:
        per = total / count
        rec = {"kernel": name, "launches_per_step": count // args.steps, "ms": round(per, 4),
               "step_ms": round(total / args.steps, 4)}
        if name in per_pair:
            fl = per_pair[name] * s.dh * pairs * s.H
            rec["tflops"] = round(fl / (per * 1e-3) / 1e12, 1)
        else:  # RoPE: read and write one tensor
            heads = s.H if name.endswith("Q") else s.Hkv
            rec["gbs"] = round(2 * s.T * heads * s.dh * 2 / (per * 1e-3) / 1e9, 1)
        kernels.append(rec)
    dom = max((k for k in kernels if "tflops" in k), key=lambda k: k["step_ms"])
    # Algorithmic HBM bytes per launch: each tensor read or written once.
    qb, kb, rowb = s.T * s.H * s.dh * 2, s.T * s.Hkv * s.dh * 2, s.T * s.H * 4
    attn_bytes = {"attention fwd": qb + 2 * kb + qb + rowb,
                  "attention bwd dQ": 3 * qb + 2 * kb + rowb + qb + 2 * rowb,
                  "attention bwd dK dV": 2 * qb + 2 * kb + 2 * rowb + 2 * kb}
    traffic, traffic_alg = _traffic_record(dom["kernel"], s.name), None
    if traffic is not None:
        traffic_alg = attn_bytes[dom["kernel"]]
    flop = 14 * s.dh * pairs * s.H
    tflops = flop / (ms * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import attention as oa
        S = s.seq_len  # the first sequence, every head
        sl = {n: inp[n][:S] for n in ("Q", "K", "V", "dO")}
        t0 = time.perf_counter()
        oa.attention_forward(sl["Q"], sl["K"], sl["V"], S, s.H, s.Hkv, s.dh, s.base)
        oa.attention_backward(sl["Q"], sl["K"], sl["V"], sl["dO"], S, s.H, s.Hkv, s.dh, s.base)
        dt = time.perf_counter() - t0
        cfl = 14 * s.dh * (S * (S + 1) / 2) * s.H
        cpu = {"value": round(cfl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _blas_threads(),
               "kind": "oracle", "seconds": round(dt, 2),
               "sample": f"the first of {s.n_seq} sequences ({S} tokens), all {s.H} query heads "
                         f"and {s.Hkv} key/value heads, fwd+bwd, numpy float64"}

    line = {
        "metric": "causal RoPE attention fwd+bwd TFLOP/s",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "launch": "hip graph" if args.graph else "eager",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q, K, V, dO)",
        "config": {"workload": s.name, "tokens": s.T, "seq_len": s.seq_len, "heads": s.H,
                   "kv_heads": s.Hkv, "head_dim": s.dh, "rope_base": s.base},
        "mfma_peak_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"kernel": dom["kernel"], "bound": "mfma", "achieved": dom["tflops"],
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_algorithmic_bytes": traffic_alg, "ms_per_launch": dom["ms"]},
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the block; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: collectives and multi-GPU runs are "
              "outside this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import gemm_online_rmsnorm_amd as lr
    from gemm_online_rmsnorm_amd.runner import BlockRun
    from gemm_online_rmsnorm_amd.work import is_memory_bound, kernel_work

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lr._lib.load()
    if args.attention == "block":
        block_attention_main(args)
        return
    if args.attention:
        attention_main(args)
        return
    s = synth.config(args.config)
    if args.vendor_gemms:
        vendor_gemms_main(args, s)
        return
    if args.tp_split:
        tp_split_main(args, s)
        return
    if args.gemm_sweep:
        gemm_sweep_main(args)
        return
    print(f"[bench] workload {s.name} T={s.T} d={s.d} r={s.r} F={s.F} D={s.D} P={s.P}",
          file=sys.stderr, flush=True)
    inputs = synth.make_inputs(s)
    run = BlockRun(s.T, s.d, s.r, s.F, s.D, s.P, s.dtype, s.eps, s.partials, inputs,
                   heads=s.heads)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        _calibration_copy(torch)

    for _ in range(args.warmup):
        run.step(stream)
    timed = _timed_step(torch, args, run.step, stream)
    torch.cuda.synchronize()

    # Timed region: K steps between events on the stream the library uses
    # (one event before the first step and one after each step).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        timed()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    ms_median = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]))

    # Per-kernel pass: the library brackets each launch with HIP events on
    # its stream; same K steps again.
    lr.profile_enable(True)
    for _ in range(args.steps):
        run.step(stream)
    torch.cuda.synchronize()
    lr.profile_enable(False)
    prof = lr.profile_collect(with_bytes=True)
    elem = 2 if s.dtype == "bf16" else 4
    work = kernel_work(s.T, s.d, s.r, s.F, elem, s.partials, s.P)
    kernels = []
    for name, count, total, nbytes in prof:
        per = total / count
        # Launches whose bytes depend on a choice made at run time (the
        # split-K sums) take the count the library recorded for them.
        fl, by = work.get(name, (0.0, nbytes / count if count else 0.0))
        kernels.append({
            "kernel": name, "launches_per_step": count // args.steps,
            "ms": round(per, 4),
            "tflops": round(fl / (per * 1e-3) / 1e12, 1) if fl else None,
            "gbs": round(by / (per * 1e-3) / 1e9, 1) if by else None,
            "bound": "hbm" if is_memory_bound(name) else "mfma",
            "step_ms": round(total / args.steps, 4),
        })
    kernel_ms = sum(k["step_ms"] for k in kernels)
    dom = max(kernels, key=lambda k: k["step_ms"])

    # Memory-bound kernels, GPU-side: a pass in which each of them is
    # enqueued HBM_REPEAT times back to back between its events, so the
    # per-launch time leaves out the launch latency of a single launch.
    lr.profile_repeat(HBM_REPEAT)
    lr.profile_enable(True)
    for _ in range(min(args.steps, 3)):
        run.step(stream)
    torch.cuda.synchronize()
    lr.profile_enable(False)
    lr.profile_repeat(1)
    hbm = []
    for name, count, total, nbytes in lr.profile_collect(with_bytes=True):
        if not is_memory_bound(name) or count == 0 or total <= 0:
            continue
        gbs = nbytes / (total * 1e-3) / 1e9
        hbm.append({"kernel": name, "us": round(1e3 * total / count, 2),
                    "bytes": round(nbytes / count), "gbs": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 3)})
    peak = MFMA_BF16_PEAK_TFLOPS if s.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    roofline = {
        "kernel": dom["kernel"],
        "bound": dom["bound"],
        "achieved": dom["tflops"] if dom["bound"] == "mfma" else dom["gbs"],
        "peak": peak if dom["bound"] == "mfma" else HBM_PEAK_GBS,
        "unit": "TFLOP/s" if dom["bound"] == "mfma" else "GB/s",
        "traffic": None,
        "ms_per_launch": dom["ms"],
    }
    # Measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    # copy-calibrated), when taken on the current kernel sources.
    roofline["traffic"] = _traffic_record(dom["kernel"], s.name)
    if roofline["traffic"] is not None:
        roofline["traffic_algorithmic_bytes"] = round(work[dom["kernel"]][1])
    roofline["frac"] = round(roofline["achieved"] / roofline["peak"], 4)

    flop_step = s.T * (s.fwd_flop_per_token() + s.bwd_flop_per_token()
                       + s.recompute_flop_per_token())
    flop_model = s.T * 3 * s.fwd_flop_per_token()
    tflops = flop_step / (ms * 1e-3) / 1e12

    cpu, par = None, None
    if not args.no_cpu_baseline:
        print("[bench] cpu_baseline: timing the fp64 oracle on a sample", file=sys.stderr,
              flush=True)
        gpu_out = run.results(host_dtype=np.float32)
        cpu, ref, rows = cpu_baseline(s, inputs, args.cpu_rows)
        # The outputs of the last step of the passes above; every step
        # recomputes them from the same inputs.
        par = parity(gpu_out, ref, rows, s.T, 1e-2 if s.dtype == "bf16" else 1e-5)
        del gpu_out, ref

    line = {
        "metric": "fwd+bwd low-rank block tokens/s + TFLOP/s as % of MI355X bf16 MFMA peak",
        "value": round(s.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4),
        "launch": "hip graph" if args.graph else "eager",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded Gaussian inputs and random-init factors of the workload's shapes)",
        "config": {"workload": f"{s.name} low-rank decoder-block linear stack, fwd+bwd",
                   "tokens": s.T, "d": s.d, "r": s.r, "d_ff": s.F, "d_norm": s.D,
                   "n_panels": s.P, "rank_share": s.partials},
        "tflops": round(tflops, 1),
        "tflops_model": round(flop_model / (ms * 1e-3) / 1e12, 1),
        "mfma_peak_frac": round(tflops / peak, 4),
        "roofline": roofline,
        "hbm_phases": hbm,
        "kernel_ms_sum": round(kernel_ms, 4),
        "wall_s": round(wall, 3),
        "parity": par,
        "cpu_baseline": cpu,
    }
    if args.kernels:
        for k in sorted(kernels, key=lambda k: -k["step_ms"]):
            print(json.dumps(k), file=sys.stderr)
    print(json.dumps(line), flush=True)
    if par is not None and not par["ok"]:
        print(f"[bench] parity FAILED: {par['tensor']} off by {par['worst']:.3e} "
              f"(tol {par['tol']})", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
