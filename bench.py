#!/usr/bin/env python3
"""SDPA-backward throughput on one MI355X.

Default workload: the GPT-2-shape problem of the cuDNN SDPA-backward sample
(B=4, H=12, S=1024, D=64, fp16, BSHD physical / BHSD logical strides, causal,
scale 1/8; cudnn-frontend notebook, problem-sizes and tensor cells).  One step
is one sdpa_bwd call: preprocess, main kernel and dQ conversion, on inputs
already resident in HBM (Q, K, V, dO drawn by synth; O and the LSE from the
library's forward, outside the timed region).  Before the W warm-up steps the
step runs untimed for 0.2 s of wall time so that the GPU's clocks have ramped
up from idle (reported as clock_ramp_s).

Prints ONE JSON line:
  value       counted TFLOP/s of the whole step: 5 matmuls of 2*Sq*Sk*D per
              head, halved for causal, divided by the measured step time;
  roofline    the main kernel's counted FLOP per launch over its average
              duration, against the MI355X dense fp16/bf16 MFMA peak of
              2516.6 TFLOP/s.  The duration comes from HIP events that the
              runtime fills with the kernel's own dispatch-packet begin and end
              timestamps (hipExtLaunchKernelGGL on the launch stream), over the
              same K steps run again; a kernel time longer than the whole step
              cannot be right and is reported as null;
  cpu_baseline the fp64 CPU oracle on the same inputs, timed on this host.

    python bench.py [--steps K] [--warmup W] [--config 2|3|4|5] [--dq-mode 0|1|2]
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
RAMP_S = 0.2          # untimed steps before the warm-up steps, in seconds of wall time
def kernel_sources(kernel: str) -> list:
    """The files a kernel's code comes from: its sources (NSA kernels also use
    the dense preprocess) and the build script, which holds the compiler flags."""
    base = ("common.h", "bwd_shared.h", "bwd.hip", "bwd_big.h", "bwd128.hip", "bwd192.hip")
    files = base + ("nsa.hip", "nsa_kv.hip") if kernel.startswith("nsa") else base
    return [os.path.join(ROOT, "sdpa_backward_fa2_amd", "csrc", f) for f in files] + [
        os.path.join(ROOT, "sdpa_backward_fa2_amd", "build.py")]


def kernel_source_hash(kernel: str = "bwd_fused8_kernel") -> str:
    h = hashlib.sha256()
    for f in kernel_sources(kernel):
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
    ap.add_argument("--deterministic", action="store_true", help="dQ mode 1 (same as --dq-mode 1)")
    ap.add_argument("--dq-mode", type=int, choices=[0, 1, 2], default=None,
                    help="0 fastest (default), 1 bitwise reproducible, 2 fp32 atomic accumulation")
    ap.add_argument("--head-dims", default=None, metavar="D,DV",
                    help="selected workload only: query/key and value head dims, e.g. 192,128 "
                         "(the NSA page's unequal head dims); default the workload's own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 256 MiB (10 launches), the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def build_inputs(cid: int, head_dims=None):
    """Device inputs and a prepared call for workload `cid` (with other head
    dims when given); also the fp64 host copies the CPU baseline needs."""
    import numpy as np
    import torch

    import sdpa_backward_fa2_amd as sb
    import synth
    wl = synth.workload(cid)
    if head_dims is not None:
        wl = synth.with_head_dims(wl, *head_dims)
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

        def prep(det):
            return sb.prepare_bwd(ts["q"], ts["k"], ts["v"], o, ts["do"], lse, wl.scale, wl.causal,
                                  deterministic=det)
        return wl, prep, host

    ts = {}
    for name, tid, H in (("q", synth.TID_Q, wl.Hq), ("k", synth.TID_K, wl.Hkv),
                         ("v", synth.TID_V, wl.Hkv), ("do", synth.TID_DO, wl.Hq)):
        bits = wl.packed_bits(tid, H)
        ts[name], host[name] = dev(bits), bits
    cu = wl.cu_seqlens()
    T = wl.T
    if wl.kind == "varlen":
        # O and the LSE from the library's packed forward (outside the timed region)
        o, lse = sb.fwd_stats_varlen(ts["q"], ts["k"], ts["v"], cu, cu, wl.scale, wl.causal)
        torch.cuda.synchronize()

        def prep(det):
            return sb.prepare_varlen(ts["q"], ts["k"], ts["v"], o, ts["do"], lse, cu, cu, wl.scale,
                                     wl.causal, deterministic=det)
        return wl, prep, host

    # selected (NSA): O and the (max, sum) statistics over the gathered keys
    # from the library's selected forward, outside the timed region
    topk_np = wl.topk()
    topk = torch.from_numpy(np.ascontiguousarray(topk_np, dtype=np.int32)).cuda()
    bs = wl.block_size
    o, m, l = sb.fwd_selected(ts["q"], ts["k"], ts["v"], topk, cu, cu, bs, wl.scale,
                              wl.extra.get("sparse_mode", 2))
    torch.cuda.synchronize()

    def prep(det):
        return sb.prepare_selected(ts["q"], ts["k"], ts["v"], o, ts["do"], (m, l), topk, cu, cu, bs,
                                   wl.scale, wl.extra.get("sparse_mode", 2), deterministic=det)
    host["topk"] = topk_np
    return wl, prep, host


def cpu_baseline(wl, host) -> dict:
    """The fp64 oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    import synth
    try:
        host_cores = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        host_cores = os.cpu_count() or 1
    blas, threads = "unknown", host_cores
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if pools:
            blas = ",".join(sorted({str(i.get("internal_api")) for i in pools}))
            threads = max(int(i.get("num_threads", 1)) for i in pools)
    except Exception:  # pragma: no cover
        pass
    x = {k: synth.decode(v, wl.dtype) if wl.kind != "dense" else v
         for k, v in host.items() if k in ("q", "k", "v", "do")}
    if wl.kind == "dense":
        units = [(b, h) for b in range(wl.B) for h in range(wl.Hkv)]
        what = "(batch, KV head) slices"

        def run(sel):
            oracle.dense_backward(x["q"], x["k"], x["v"], x["do"], wl.scale, wl.causal, heads=sel)

        def share(sel):
            return len(sel) / len(units)
    elif wl.kind == "varlen":
        cu = wl.cu_seqlens()
        units = list(range(len(cu)))
        what = "sequences"

        def run(sel):
            oracle.varlen_backward(x["q"], x["k"], x["v"], x["do"], cu, cu, wl.scale, wl.causal, seqs=sel)

        lens = np.diff(np.concatenate([[0], cu])).astype(np.float64)

        def share(sel):
            return float(np.sum(lens[sel] ** 2) / np.sum(lens ** 2))
    else:
        cu = wl.cu_seqlens()
        units = [0]
        what = "the whole problem"

        def run(sel):
            oracle.selected_backward(x["q"], x["k"], x["v"], x["do"], host["topk"], cu, cu,
                                     wl.block_size, wl.scale, wl.extra.get("sparse_mode", 2))

        def share(sel):
            return 1.0
    # size the sample: time one unit, then take enough units for ~10 s per repetition
    t0 = time.perf_counter()
    run(units[:1])
    t_one = time.perf_counter() - t0
    n = int(min(len(units), max(1, math.ceil(10.0 / max(t_one, 1e-3)))))
    reps = 3 if n == len(units) and t_one * n < 8 else 1
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        run(units[:n])
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    flops = wl.counted_flops() * share(units[:n])
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "host_cores": int(host_cores), "blas": blas, "blas_threads": int(threads),
            "sample": f"{n} of {len(units)} {what} of the same problem, fp64 numpy oracle, "
                      f"median of {reps} run(s), {t:.2f} s per run"}


# Share of the counted contractions (S, dP, dV, dK, dQ) each kernel performs,
# keyed by (kernel, dQ formed without atomics); recomputed S and dP in the
# query-outer dQ kernels are not counted.
KERNEL_FLOP_SHARE = {
    ("bwd_fused8_kernel", True): 1.0, ("bwd_fused2_kernel", True): 1.0,
    ("bwd_main_kernel", False): 1.0, ("bwd_main_kernel", True): 0.8, ("bwd_dq8_kernel", True): 0.2,
    ("nsa_kv_kernel", True): 0.8, ("nsa_dq_kernel", True): 0.2,
}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, if they were taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    e = rec.get(kernel, {}).get(workload)
    if not e or e.get("source_hash") != kernel_source_hash(kernel):
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
    mode = args.dq_mode if args.dq_mode is not None else (1 if args.deterministic else 0)
    head_dims = None
    if args.head_dims:
        head_dims = tuple(int(x) for x in args.head_dims.split(","))
        if args.config != 5 or len(head_dims) != 2:
            sys.exit("--head-dims D,DV applies to the selected workload (--config 5) only")
    wl, prep, host = build_inputs(args.config, head_dims)
    call, outs = prep(mode)
    # Clock ramp: from idle the GPU takes some 50 ms to reach its steady
    # clocks (measured on MI355X: the GPT-2-shape step runs 58 -> 48 -> 42 us
    # over the first 40 ms, then holds), so the step runs untimed for RAMP_S
    # of wall time before the W warm-up steps; the K timed steps then see the
    # clocks a running training loop sees.
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < RAMP_S:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    ramp_s = time.perf_counter() - t_ramp
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

    # per-kernel durations: the same K steps again, each launch carrying an event
    # pair filled with its dispatch packet's begin and end timestamps
    with sb.KernelTimer() as kt:
        for _ in range(args.steps):
            call()
    torch.cuda.synchronize()
    kernels = {k: {"avg_us": 1e3 * t / n, "launches": n} for k, (t, n) in kt.result.items()}
    # the dominant kernel, with the counted contractions it performs
    main_name = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    atomic = mode == 2 and wl.D == 128 and wl.kind != "selected"
    share = KERNEL_FLOP_SHARE.get((main_name, not atomic), 0.0)
    main_us = kernels[main_name]["avg_us"]
    per_launch = flops * share * args.steps / kernels[main_name]["launches"]
    # a kernel of the step cannot take longer than the step
    sane = main_us * 1e-3 <= ms * 1.001
    achieved = per_launch / (main_us * 1e-6) / 1e12 if sane else None
    workload_name = f"config{args.config}" + (f"_d{wl.D}_dv{wl.Dv}" if head_dims else "")
    roofline = {"bound": "mfma", "kernel": main_name, "achieved": achieved,
                "peak": PEAK_MFMA_16BIT_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_MFMA_16BIT_TFLOPS if sane else None,
                "traffic": traffic_for(main_name, workload_name)}
    if wl.kind == "dense":
        cfg = {"workload": wl.name, "B": wl.B, "H": wl.Hq, "S": wl.S, "D": wl.D, "causal": wl.causal,
               "layout": wl.layout}
    else:
        cfg = {"workload": wl.name, "T": wl.T, "sequences": len(wl.lengths), "Hq": wl.Hq, "Hkv": wl.Hkv,
               "D": wl.D, "causal": wl.causal}
        if wl.Dv != wl.D:
            cfg["Dv"] = wl.Dv
        if wl.kind == "selected":
            cfg.update(block_size=wl.block_size, block_count=wl.block_count)
    cfg.update(dq_mode=mode, counted_gflop=flops / 1e9)

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "clock_ramp_s": round(ramp_s, 3), "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": cfg,
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
