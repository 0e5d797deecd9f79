#!/usr/bin/env python
"""Benchmark of one MI355X's share of the flash all-reduce (quantize -> reduce-scatter -> all-gather
dequantize + residual-add + RMSNorm), on synthetic inputs already resident in HBM.

A step is the whole emulated all-reduce of one batch on one GPU: all R ranks' group quantization (one
launch), all R shards' fixed-order dequant-reduce-requant (one launch), and the all-gather dequantize
with the fused RMSNorm epilogue (one launch).  Steps are replayed from a HIP graph; each step uses its
own buffer set, and the sets together exceed twice the 256 MB last-level cache, so every step reads
from HBM ("cold").  value = algorithmic bytes per step / time per step.

Prints one JSON line.  --gpus N > 1 is refused: this build runs on one GPU.
"""
import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused quant-reduce-RMSNorm effective GB/s (% HBM peak) + µs per call"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=2, help="two-step workload: 1, 2 or 3")
    ap.add_argument("--warm", action="store_true", help="reuse one buffer set (cache-resident)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=0, help="graph replays per kernel timing (0 = auto)")
    return ap.parse_args()


def cpu_baseline(cfg, seconds):
    """The oracle (single-threaded C++) on the same workload, whole steps repeated for about `seconds`."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import oracle
    from tensor_all_reduce_amd import bytes_model as bm, datagen as dg
    if cfg.n > (1 << 22):  # the 70B prefill step takes minutes on one core: time one row block
        T = max(cfg.R, (1 << 22) // cfg.H // cfg.R * cfg.R)
        sample = f"{T} of {cfg.T} tokens x all {cfg.R} ranks, whole steps repeated"
    else:
        T = cfg.T
        sample = f"the whole step ({cfg.R} ranks x {cfg.T} x {cfg.H}), repeated"
    n = T * cfg.H
    parts = [dg.partial(cfg, r, n) for r in range(cfg.R)]
    res, gam = dg.residual(cfg, n), dg.gamma(cfg)
    step_bytes = sum(bm.total(v) for v in bm.two_step_whole(cfg.R, T, cfg.H, cfg.bits_rs, cfg.bits_ag,
                                                             cfg.group).values())
    oracle.lib()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.two_step(parts, cfg.bits_rs, cfg.bits_ag, cfg.group, residual=res, gamma=gam, eps=cfg.eps,
                        hidden=cfg.H, plain=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(step_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": sample + f" {reps}x in {el:.1f} s; single-threaded C++ (g++ -O2 -ffp-contract=off)",
            "us_per_step": round(el / reps * 1e6, 1), "host_cpu": platform.processor() or platform.machine(),
            "host_cores": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build emulates the R ranks on one GPU "
              "(inter-GPU transfers are local HBM buffers); run with --gpus 1", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    from tensor_all_reduce_amd import _lib, bytes_model as bm, datagen as dg
    from tensor_all_reduce_amd.flash_allreduce import TwoStepAllReduce

    cfg = dg.CONFIGS[args.config]
    assert cfg.kind == "two_step", "the benchmark's metric is the quantized two-step path"
    dev = torch.device("cuda:0")
    R, T, H, G, b1, b2 = cfg.R, cfg.T, cfg.H, cfg.group, cfg.bits_rs, cfg.bits_ag
    calls = bm.two_step_whole(R, T, H, b1, b2, G)
    step_bytes = sum(bm.total(v) for v in calls.values())

    # ---- inputs, resident in HBM before timing
    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    parts0 = up(np.stack(dg.partials(cfg)))
    res0, gam = up(dg.residual(cfg)), up(dg.gamma(cfg))
    set_bytes = step_bytes
    nsets = 1 if args.warm else max(1, math.ceil(2 * MALL_BYTES / set_bytes))
    sets = []
    for k in range(nsets):
        p = TwoStepAllReduce(R, T, H, b1, b2, G, device=dev, parts=parts0.clone() if k else parts0)
        res = res0.clone() if k else res0
        out = torch.empty(cfg.n, dtype=torch.int16, device=dev)
        rout = torch.empty(cfg.n, dtype=torch.int16, device=dev)
        sets.append((p, p.make_norm(gam, out, residual=res, residual_out=rout, eps=cfg.eps), (res, out, rout)))
    torch.cuda.synchronize()

    def step(k):
        p, norm, _ = sets[k]
        p.run(norm=norm)

    # warm-up (eager, then graph)
    for k in range(min(args.warmup, nsets)):
        step(k)
    torch.cuda.synchronize()
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all):
        for k in range(nsets):
            step(k)
    tail = args.steps % nsets
    g_tail = None
    if tail:
        g_tail = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_tail):
            for k in range(tail):
                step(k)
    for _ in range(max(1, args.warmup // nsets)):
        g_all.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly args.steps steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps // nsets):
        g_all.replay()
    if g_tail is not None:
        g_tail.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # ---- per-call durations: each call alone, replayed from a graph over the same buffer sets
    def time_call(fn, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(nsets):
                fn(k)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * nsets)  # microseconds per launch

    reps = args.kernel_reps or max(1, args.steps // nsets)
    fns = {
        "quantize": lambda k: sets[k][0].quantize(),
        "reduce_shard": lambda k: sets[k][0].reduce_scatter(),
        "gather_norm": lambda k: sets[k][0].all_gather(norm=sets[k][1]),
    }
    per_call = {}
    for name, fn in fns.items():
        us = time_call(fn, reps)
        by = bm.total(calls[name])
        per_call[name] = {"us": round(us, 3), "bytes": by, "GB/s": round(by / (us * 1e-6) / 1e9, 1),
                          "frac_hbm": round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    dom = max(per_call, key=lambda k: per_call[k]["us"])

    # ---- practical copy ceiling (1 GiB each way)
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty(nb, dtype=torch.uint8, device=dev)
    _lib.fc_copy(src, dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        _lib.fc_copy(src, dst)
    b.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nb * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "R": R, "T": T, "H": H, "bits_rs": b1, "bits_ag": b2, "group": G,
                   "mode": "whole emulated all-reduce on one GPU", "cache": "warm" if args.warm else "cold",
                   "buffer_sets": nsets, "launch": "hip graph, 3 kernels per step"},
        "us_per_step": round(ms_step * 1e3, 3), "bytes_per_step": step_bytes,
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "copy_ceiling_GBps": round(copy_gbps, 1), "pct_copy_ceiling": round(100 * value / copy_gbps, 2),
        "calls": per_call,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": per_call[dom]["GB/s"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": per_call[dom]["frac_hbm"], "traffic": None},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
