"""Benchmark of the Agent Attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full forward (pool -> aggregate -> broadcast) over one batch of
the workload.  Inputs are synthetic, generated on the device, and rotate over
enough buffer sets (>= 1 GiB in total) that each step reads its Q, K, V from
HBM rather than from the 256 MB Infinity Cache.  The K timed steps are
captured once into a HIP graph and replayed, bracketed by device
synchronisations; every kernel launch of the forward is also timed on its
stream with HIP events in an eager run of the same K steps, which gives the
per-launch kernel duration used for the roofline.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores


def algorithmic_bytes(wl) -> int:
    """Q, K, V read once and O written once (plus caller agents read once)."""
    b = 4 * wl.B * wl.H * wl.N * wl.d * wl.es
    if wl.supplied_agents:
        b += wl.B * wl.H * wl.k * wl.d * wl.es
    return b


def algorithmic_flops(wl) -> int:
    """Four N x k x d products per head: 2 * 4 * N * k * d."""
    return 8 * wl.B * wl.H * wl.N * wl.k * wl.d


def cpu_baseline(wl, min_seconds=10.0):
    """The float64 oracle timed on the host cores on the same workload shape."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle
    from efficient_attention_vision_amd import inputs

    inp = inputs.make_inputs(wl, 0, "iid")
    A = None if inp.A is None else inp.A.exact
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale, A=A)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds and reps >= 2:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    tokens = wl.B * wl.H * wl.N * reps
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full forwards of the {wl.name} workload (float64 numpy) in "
                      f"{el:.1f} s on {os.cpu_count()} visible host CPUs ({platform.processor() or platform.machine()})",
            "seconds": el}


COPY_BYTES = 64 << 20


def copy_calibration(torch, steps):
    """Plain device-to-device copies of COPY_BYTES each, over rotating
    buffers (> 1 GiB in total), so that an HBM counter read per dispatch can
    be divided by the known COPY_BYTES read and written."""
    dev = torch.device("cuda:0")
    n = COPY_BYTES // 4
    bufs = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(20)]
    for i in range(steps):
        bufs[(2 * i + 1) % 20].copy_(bufs[(2 * i) % 20])
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                                           "copies": steps}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pvt_stage1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only plain device copies of known size (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads are independent: each GPU would run this same forward on its share of B*H)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch, args.steps)
        return
    import efficient_attention_vision_amd as eav
    from efficient_attention_vision_amd import _binding, inputs

    wl = inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    shape = (wl.B, wl.H, wl.N, wl.d)
    set_bytes = algorithmic_bytes(wl)
    R = max(2, min(args.steps, math.ceil((1 << 30) / set_bytes)))
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    sets = []
    for _ in range(R):
        q, k, v = (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
                   .mul_(wl.sigma).to(dt) for _ in range(3))
        a = (torch.randn((wl.B, wl.H, wl.k, wl.d), generator=gen, device=dev).to(dt)
             if wl.supplied_agents else None)
        sets.append((q, k, v, a, torch.empty_like(q)))
    need = _binding.agent_attn_workspace_bytes(wl.B, wl.H, wl.h, wl.w, wl.d, wl.s,
                                               0 if wl.dtype == "f32" else 1)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, a, o = sets[i % R]
        eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale, agents=a, out=o,
                               workspace=ws)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # eager run: every launch bracketed by events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    launch_ms_sorted = sorted(launch_ms)
    kernel_us = 1e3 * sum(launch_ms) / len(launch_ms)
    kernel_us_median = 1e3 * launch_ms_sorted[len(launch_ms) // 2]

    # graph of exactly K steps, replayed once in the timed region
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(args.steps):
                step(i)
    stream.wait_stream(side)
    g.replay()   # warm replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = 1e3 * (t1 - t0) / args.steps

    tokens = wl.B * wl.H * wl.N
    value = tokens / (ms_per_step * 1e-3)
    abytes = algorithmic_bytes(wl)
    aflops = algorithmic_flops(wl)
    achieved_gbs = abytes / (kernel_us * 1e-6) / 1e9
    achieved_tflops = aflops / (kernel_us * 1e-6) / 1e12
    if wl.k >= 256:
        roof = {"bound": "mfma", "achieved": achieved_tflops, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved_tflops / BF16_PEAK_TFLOPS, "traffic": None}
    else:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": None}
    line = {
        "metric": "agent-attn fwd tokens/s (B*H*N/s) + achieved HBM GB/s at N=3136,k=49 bf16",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "grid": [wl.h, wl.w], "N": wl.N,
                   "d": wl.d, "agents": wl.k, "agent_grid": [wl.s, wl.s],
                   "supplied_agents": wl.supplied_agents, "rotating_sets": R},
        "roofline": roof,
        "kernel_us_mean": kernel_us,
        "kernel_us_median": kernel_us_median,
        "achieved_hbm_gbs": achieved_gbs,
        "achieved_tflops": achieved_tflops,
        "algorithmic_bytes": abytes,
        "algorithmic_flops": aflops,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, args.cpu_seconds)
        cb.pop("seconds", None)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
