#!/usr/bin/env python3
"""SDPA-backward throughput on one MI355X.

Default workload: the GPT-2-shape problem of the cuDNN SDPA-backward sample
(B=4, H=12, S=1024, D=64, fp16, BSHD physical / BHSD logical strides, causal,
scale 1/8; cudnn-frontend notebook, problem-sizes and tensor cells).  One step
is one sdpa_bwd call: preprocess, main kernel and dQ conversion, on inputs
already resident in HBM (Q, K, V, dO drawn by synth; O and the LSE from the
library's forward, outside the timed region).

Prints ONE JSON line:
  value       counted TFLOP/s of the whole step: 5 matmuls of 2*Sq*Sk*D per
              head, halved for causal, divided by the measured step time;
  roofline    the main kernel's counted FLOP per launch over its average
              duration (HIP events around each launch on its stream), against
              the MI355X dense fp16/bf16 MFMA peak of 2516.6 TFLOP/s;
  cpu_baseline the fp64 CPU oracle on the same inputs, timed on this host.

    python bench.py [--steps K] [--warmup W] [--config 2|3|4|5] [--deterministic]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SDPA-backward TFLOP/s on 1 MI355X (GPT-2 shape, causal); % of MFMA peak"
PEAK_MFMA_16BIT_TFLOPS = 2516.6      # 256 CU x 4096 FLOP/clk/CU x 2.4 GHz, dense fp16/bf16
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "sdpa_backward_fa2_amd", "csrc", f)
                  for f in ("common.h", "bwd.hip", "nsa.hip")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        if os.path.exists(f):
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5])
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 256 MiB (10 launches), the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def build_inputs(cid: int):
    """Device inputs and a prepared call for workload `cid`; also the fp64
    host copies the CPU baseline needs."""
    import numpy as np
    import torch

    import sdpa_backward_fa2_amd as sb
    import synth
    wl = synth.workload(cid)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[wl.dtype]

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(dt)

    host = {}
    if wl.kind == "dense":
        ts = {}
        for name, tid, H in (("q", synth.TID_Q, wl.Hq), ("k", synth.TID_K, wl.Hkv),
                             ("v", synth.TID_V, wl.Hkv), ("do", synth.TID_DO, wl.Hq)):
            phys = synth.normal_bits(wl.dense_physical_shape(H), wl.dtype, cid, tid)
            t = dev(phys)
            x = synth.decode(phys, wl.dtype)
            if wl.layout == "bshd":
                t, x = t.permute(0, 2, 1, 3), x.transpose(0, 2, 1, 3)
            ts[name], host[name] = t, x
        o, lse = sb.fwd_stats(ts["q"], ts["k"], ts["v"], wl.scale, wl.causal)
        torch.cuda.synchronize()
        call, outs = sb.prepare_bwd(ts["q"], ts["k"], ts["v"], o, ts["do"], lse, wl.scale,
                                    wl.causal, deterministic=False)
        return wl, call, outs, host, (ts, o, lse)
    raise SystemExit(f"config {cid}: bench line not implemented yet")


def cpu_baseline(wl, host) -> dict:
    """The fp64 oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    B, Hq = wl.B, wl.Hq
    heads = [(b, h) for b in range(B) for h in range(wl.Hkv)]
    # size the sample: time one head, then take enough heads for ~10 s per repetition
    t0 = time.perf_counter()
    oracle.dense_backward(host["q"], host["k"], host["v"], host["do"], wl.scale, wl.causal, heads=heads[:1])
    t_head = time.perf_counter() - t0
    n = int(min(len(heads), max(1, math.ceil(10.0 / max(t_head, 1e-3)))))
    reps = 3 if n == len(heads) and t_head * n < 8 else 1
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.dense_backward(host["q"], host["k"], host["v"], host["do"], wl.scale, wl.causal,
                              heads=heads[:n])
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    flops = wl.counted_flops() * n / len(heads)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {len(heads)} (batch, head) slices of the same problem, fp64 numpy "
                      f"oracle, median of {reps} run(s), {t:.2f} s per run"}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, if they were taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    e = rec.get(kernel, {}).get(workload)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this SDPA backward has no multi-GPU path in this build.", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 10}))
        return
    import sdpa_backward_fa2_amd as sb
    sb.load()
    wl, call, outs, host, keep = build_inputs(args.config)
    if args.deterministic:
        ts, o, lse = keep
        call, outs = sb.prepare_bwd(ts["q"], ts["k"], ts["v"], o, ts["do"], lse, wl.scale, wl.causal,
                                    deterministic=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    flops = wl.counted_flops()
    value = flops / (ms * 1e-3) / 1e12

    # per-kernel durations: the same K steps again with HIP events around every launch
    with sb.KernelTimer() as kt:
        for _ in range(args.steps):
            call()
    torch.cuda.synchronize()
    kernels = {k: {"avg_us": 1e3 * t / n, "launches": n} for k, (t, n) in kt.result.items()}
    main_name = "bwd_main_kernel"
    main_us = kernels[main_name]["avg_us"]
    achieved = flops / (main_us * 1e-6) / 1e12
    workload_name = f"config{args.config}"
    roofline = {"bound": "mfma", "kernel": main_name, "achieved": achieved,
                "peak": PEAK_MFMA_16BIT_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_MFMA_16BIT_TFLOPS,
                "traffic": traffic_for(main_name, workload_name)}

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.Hq, "S": wl.S, "D": wl.D,
                   "causal": wl.causal, "layout": wl.layout, "deterministic": args.deterministic,
                   "counted_gflop": flops / 1e9},
        "pct_of_mfma_peak": 100.0 * value / PEAK_MFMA_16BIT_TFLOPS,
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
