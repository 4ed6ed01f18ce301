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
FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X fp32 vector arithmetic
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "efficient_attention_vision_amd", "csrc")
FUSED_KERNEL = "agent_mfma_kernel"

# rocprofv3 runs whose output the summaries below are made from (run from
# /tmp with TMPDIR=/tmp; R = repository root, OUT = the folder for profiler output)
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt_{w} -o run "
             "-- python3 $R/bench.py --workload {w} --no-cpu-baseline --steps 50 --warmup 5")
PMC_CMD = ("timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d $OUT/{d} -o run "
           "-- python3 $R/bench.py {a}")


def _strip_comments(src: str) -> str:
    """C/C++ source without its comments (string and character literals kept)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":   # literal: copy through its closing quote
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return "".join(out)


def kernel_sources_sha256() -> str:
    """Hash of the code (comments stripped) the forward's fused kernel is
    built and launched from (its kernels, their instances, the host library
    that plans its launches, the ABI header): HBM counters taken on older
    code are not reported."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted([os.path.join(CSRC, n) for n in ("common.hpp", "kernels_mfma.hpp",
                                                     "agent_attn.hip")]
                   + glob.glob(os.path.join(CSRC, "mfma_dc*.hip")))
    files.append(os.path.join(ROOT, "include", "agent_attn.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_strip_comments(fh.read()).encode())
    return h.hexdigest()


def counters_file(wl_name: str) -> str:
    return os.path.join(PROFILES, f"{FUSED_KERNEL}_{wl_name}_hbm_counters.md")


def read_key_values(path):
    out = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip().lstrip("-* ").strip()
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip().strip("`")] = v.strip().strip("`")
    return out


def measured_traffic(wl_name: str):
    """HBM bytes per launch of the fused kernel from the committed counter
    summary, or None when there is none or the kernel has changed since."""
    path = counters_file(wl_name)
    if not os.path.exists(path):
        return None
    kv = read_key_values(path)
    if kv.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_means(csv_path, name_part):
    import csv
    vals = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if name_part in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def write_counter_summary(wl, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """profiles/<kernel>_<workload>_hbm_counters.md from four rocprofv3 --pmc
    runs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the fused kernel,
    each scaled by what the same counter reads for plain copies of
    COPY_BYTES."""
    def one(d, name):
        m, n = _counter_means(os.path.join(d, "run_counter_collection.csv"), name)
        return m, n
    f_k, nf = one(fetch_dir, FUSED_KERNEL)
    w_k, nw = one(write_dir, FUSED_KERNEL)
    f_c, _ = one(copy_fetch_dir, "copyBuffer")
    w_c, _ = one(copy_write_dir, "copyBuffer")
    kib = COPY_BYTES / 1024
    f_scale = kib / f_c["FETCH_SIZE"]
    w_scale = kib / w_c["WRITE_SIZE"]
    fetch_b = f_k["FETCH_SIZE"] * 1024 * f_scale
    write_b = w_k["WRITE_SIZE"] * 1024 * w_scale
    total = int(round(fetch_b + write_b))
    alg = algorithmic_bytes(wl)
    rows = [
        f"# HBM counters: {FUSED_KERNEL}, workload {wl.name}",
        "",
        f"Workload: B={wl.B} H={wl.H} grid {wl.h}x{wl.w} (N={wl.N}) d={wl.d} k={wl.k} {wl.dtype}.",
        "Commands (from /tmp with TMPDIR=/tmp, R = repository root, OUT = profiler output folder), one counter per run:",
        "",
        "    " + PMC_CMD.format(c="FETCH_SIZE", d=os.path.basename(fetch_dir),
                                a=f"--workload {wl.name} --no-cpu-baseline --steps 10 --warmup 2"),
        "    " + PMC_CMD.format(c="WRITE_SIZE", d=os.path.basename(write_dir),
                                a=f"--workload {wl.name} --no-cpu-baseline --steps 10 --warmup 2"),
        "    " + PMC_CMD.format(c="FETCH_SIZE", d=os.path.basename(copy_fetch_dir),
                                a="--copy-calibration --steps 10"),
        "    " + PMC_CMD.format(c="WRITE_SIZE", d=os.path.basename(copy_write_dir),
                                a="--copy-calibration --steps 10"),
        "    python3 bench.py --workload " + wl.name + " --pmc-summary <the four -d folders>",
        "",
        "Calibration: plain device copies (`__amd_rocclr_copyBuffer`) of "
        f"{COPY_BYTES} bytes read and written per dispatch.",
        "",
        f"- copy FETCH_SIZE KiB per dispatch: {f_c['FETCH_SIZE']:.1f}",
        f"- copy WRITE_SIZE KiB per dispatch: {w_c['WRITE_SIZE']:.1f}",
        f"- fetch_scale: {f_scale:.4f}",
        f"- write_scale: {w_scale:.4f}",
        f"- fused kernel dispatches sampled: {nf.get('FETCH_SIZE', 0)} / {nw.get('WRITE_SIZE', 0)}",
        f"- fused FETCH_SIZE KiB per dispatch: {f_k['FETCH_SIZE']:.1f}",
        f"- fused WRITE_SIZE KiB per dispatch: {w_k['WRITE_SIZE']:.1f}",
        f"- fetch_bytes_per_launch: {int(round(fetch_b))}",
        f"- write_bytes_per_launch: {int(round(write_b))}",
        f"- traffic_bytes_per_launch: {total}",
        f"- algorithmic_bytes_per_launch: {alg}",
        f"- traffic / algorithmic: {total / alg:.3f}",
        f"- kernel_sources_sha256: {kernel_sources_sha256()}",
        "",
    ]
    path = counters_file(wl.name)
    with open(path, "w") as fh:
        fh.write("\n".join(rows))
    print(path)


def write_trace_summary(wl, trace_dir):
    """profiles/<kernel>_<workload>_kernel_trace.md from a rocprofv3
    --kernel-trace --stats run of this benchmark."""
    import csv
    import statistics
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    trace = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv")))
             if FUSED_KERNEL in r["Kernel_Name"]]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace]
    starts = [int(r["Start_Timestamp"]) for r in trace]
    n = len(dur)
    rows = [
        f"# Kernel trace: {FUSED_KERNEL}, workload {wl.name}",
        "",
        f"Workload: B={wl.B} H={wl.H} grid {wl.h}x{wl.w} (N={wl.N}) d={wl.d} k={wl.k} {wl.dtype}.",
        "Command (from /tmp with TMPDIR=/tmp, R = repository root, OUT = profiler output folder):",
        "",
        "    " + TRACE_CMD.format(w=wl.name),
        "    python3 bench.py --workload " + wl.name + " --trace-summary $OUT/kt_" + wl.name,
        "",
        "The run makes 5 warm-up launches, 50 event-bracketed eager launches, then a graph of",
        "50 launches replayed twice.",
        "",
        "| kernel | calls | average ns | min ns | max ns |",
        "|---|---|---|---|---|",
    ]
    for r in stats[:8]:
        name = r["Name"]
        name = name if len(name) < 70 else name[:67] + "..."
        rows.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                    f"{r['MaxNs']} |")
    if n:
        k = trace[0]
        rows += [
            "",
            f"- {FUSED_KERNEL} launches: {n}; grid {k['Grid_Size_X']} threads, workgroup "
            f"{k['Workgroup_Size_X']}, VGPR {k['VGPR_Count']}, scratch {k['Scratch_Size']} B",
            f"- average duration, all launches: {statistics.mean(dur):.2f} us",
            f"- average duration, graph-replayed launches (last {min(100, n)}): "
            f"{statistics.mean(dur[-100:]):.2f} us",
        ]
        if n > 100:
            gaps = [(starts[i + 1] - starts[i]) / 1e3 for i in range(n - 100, n - 1)]
            rows.append(f"- median start-to-start in the graph replays: {statistics.median(gaps):.2f} us")
    path = os.path.join(PROFILES, f"{FUSED_KERNEL}_{wl.name}_kernel_trace.md")
    with open(path, "w") as fh:
        fh.write("\n".join(rows) + "\n")
    print(path)


SIMD_COUNT = 1024   # MI355X: 256 CUs x 4 SIMDs


def write_mfma_summary(wl, pmc_dir, trace_dir):
    """profiles/<kernel>_<workload>_mfma_busy.md from a rocprofv3 --pmc run of
    the derived counter MfmaUtil (matrix-core busy cycles summed over the SIMDs
    / (GPU active cycles x SIMDs)) and the kernel trace of the same workload,
    which gives the flop-based utilisation beside it."""
    import csv
    import statistics
    m, n = _counter_means(os.path.join(pmc_dir, "run_counter_collection.csv"), FUSED_KERNEL)
    trace = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv")))
             if FUSED_KERNEL in r["Kernel_Name"]]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace][-100:]
    us = statistics.mean(dur)
    flops = algorithmic_flops(wl)
    util_flop = flops / (us * 1e-6) / (BF16_PEAK_TFLOPS * 1e12)
    busy = m.get("MfmaUtil")
    rows = [
        f"# Matrix-core busy: {FUSED_KERNEL}, workload {wl.name}",
        "",
        f"Workload: B={wl.B} H={wl.H} grid {wl.h}x{wl.w} (N={wl.N}) d={wl.d} k={wl.k} {wl.dtype}.",
        "Commands (from /tmp with TMPDIR=/tmp, R = repository root, OUT = profiler output folder):",
        "",
        "    " + PMC_CMD.format(c="MfmaUtil", d=os.path.basename(pmc_dir),
                                a=f"--workload {wl.name} --no-cpu-baseline --steps 10 --warmup 2"),
        "    " + TRACE_CMD.format(w=wl.name),
        f"    python3 bench.py --workload {wl.name} --mfma-summary <the two -d folders>",
        "",
        "MfmaUtil is rocprofv3's derived counter: SQ_VALU_MFMA_BUSY_CYCLES summed over the",
        f"SIMDs / (GRBM_GUI_ACTIVE x {SIMD_COUNT} SIMDs) x 100.  Busy cycles cover every",
        "matrix-core instruction the kernel issues (the lo halves of hi + lo operand pairs and",
        "the row-sum products against a ones operand included); the flop-based figure counts",
        "only the algorithmic 8 N k d per head.",
        "",
        f"- fused kernel dispatches sampled: {n.get('MfmaUtil', 0)}",
        f"- MfmaUtil per dispatch (percent): {busy:.2f}" if busy is not None else "- MfmaUtil: absent",
        f"- kernel duration (graph-replayed launches of the trace): {us:.2f} us",
        f"- algorithmic flop per launch (8 N k d per head): {flops}",
        f"- flop-based utilisation of the {BF16_PEAK_TFLOPS:.0f} TFLOP/s dense bf16 peak: "
        f"{100 * util_flop:.2f} %",
        f"- kernel_sources_sha256: {kernel_sources_sha256()}",
        "",
    ]
    path = os.path.join(PROFILES, f"{FUSED_KERNEL}_{wl.name}_mfma_busy.md")
    with open(path, "w") as fh:
        fh.write("\n".join(rows))
    print(path)


PASS_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/{d}_{w} -o run "
            "-- python3 $R/bench.py --workload {w} --no-cpu-baseline --{m} --steps 20 --warmup 2")
PASS_NAMES = {"backward": ("bwd_passes", "ktb"), "projections": ("module_projections", "ktp")}


def write_passes_summary(wl, mode, trace_dir):
    """profiles/<path>_<workload>_kernel_trace.md: the library's kernels of a
    multi-launch path (the backward, or the module with projections), from a
    rocprofv3 --kernel-trace --stats run of this benchmark in that mode."""
    import csv
    name, tag = PASS_NAMES[mode]
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    ours = [r for r in stats if "aa::" in r["Name"]]
    rows = [
        f"# Kernel trace: {mode} path, workload {wl.name}",
        "",
        f"Workload: B={wl.B} H={wl.H} grid {wl.h}x{wl.w} (N={wl.N}) d={wl.d} k={wl.k} {wl.dtype}.",
        "Command (from /tmp with TMPDIR=/tmp, R = repository root, OUT = profiler output folder):",
        "",
        "    " + PASS_CMD.format(d=tag, w=wl.name, m=mode),
        f"    python3 bench.py --workload {wl.name} --passes-summary {mode} "
        f"$OUT/{tag}_{wl.name}",
        "",
        "The run makes 2 warm-up steps, 20 event-bracketed eager steps, then a graph of 20",
        "steps replayed twice (62 steps); a kernel launched once per agent chunk (chunks of",
        "64 agents) runs several times per step.",
        "",
        "| kernel | calls | per step | average us | min us | max us |",
        "|---|---|---|---|---|---|",
    ]
    steps = min(int(r["Calls"]) for r in ours) if ours else 1
    total = 0.0
    for r in ours:
        nm = r["Name"].split("(")[0].replace("void ", "")
        nm = nm if len(nm) < 70 else nm[:67] + "..."
        avg = float(r["AverageNs"]) / 1e3
        per = int(r["Calls"]) / steps
        total += avg * per
        rows.append(f"| `{nm}` | {r['Calls']} | {per:g} | {avg:.1f} | "
                    f"{int(r['MinNs']) / 1e3:.1f} | {int(r['MaxNs']) / 1e3:.1f} |")
    rows += ["", f"- sum of the kernel durations of one step: {total:.1f} us"]
    path = os.path.join(PROFILES, f"{name}_{wl.name}_kernel_trace.md")
    with open(path, "w") as fh:
        fh.write("\n".join(rows) + "\n")
    print(path)


def algorithmic_bytes(wl) -> int:
    """Q, K, V read once and O written once (plus caller agents read once)."""
    b = 4 * wl.B * wl.H * wl.N * wl.d * wl.es
    if wl.supplied_agents:
        b += wl.B * wl.H * wl.k * wl.d * wl.es
    return b


def algorithmic_flops(wl) -> int:
    """Four N x k x d products per head: 2 * 4 * N * k * d."""
    return 8 * wl.B * wl.H * wl.N * wl.k * wl.d


def cpu_baseline(wl, min_seconds=10.0, module=False):
    """The float64 oracle timed on the host cores on the same workload shape
    (with the module terms when `module`)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle
    from efficient_attention_vision_amd import inputs

    inp = inputs.make_inputs(wl, 0, "iid")
    A = None if inp.A is None else inp.A.exact
    mt = inputs.make_module_terms(wl, 0) if module else {}
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(inp.Q.exact, inp.K.exact, inp.V.exact, wl.h, wl.w, wl.s, wl.scale, A=A,
                       **mt)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds and reps >= 2:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    tokens = wl.B * wl.H * wl.N * reps
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full forwards of the {wl.name} workload (float64 numpy) in "
                      f"{el:.1f} s with {threads} BLAS threads on {os.cpu_count()} visible host CPUs ({cpu})",
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
    ap.add_argument("--layout", choices=("bhnd", "bnhd"), default="bhnd",
                    help="q/k/v/out as dense [B,H,N,d] (default) or as [B,N,H,d] storage "
                         "(strided views, as a head-split projection leaves them)")
    ap.add_argument("--module", action="store_true",
                    help="time the full module forward: agent biases in both attentions and "
                         "the depth-wise 3x3 convolution of V (agent_attn_forward_module)")
    ap.add_argument("--projections", action="store_true",
                    help="time the attention module on token features: q/k/v projection, the "
                         "module forward (biases, DWC) and the output projection "
                         "(agent_attn_module_forward)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (agent_attn_backward: gradients of q, k, v "
                         "from the output gradient, forward recomputed inside)")
    ap.add_argument("--dtype", choices=("bf16", "f16"), default=None,
                    help="16-bit element type of the tensors (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only plain device copies of known size (for scaling HBM counters)")
    ap.add_argument("--pmc-summary", nargs=4, metavar="DIR",
                    help="write the HBM counter summary of --workload from four rocprofv3 --pmc "
                         "output folders (kernel FETCH_SIZE, kernel WRITE_SIZE, copy FETCH_SIZE, "
                         "copy WRITE_SIZE) and exit")
    ap.add_argument("--passes-summary", nargs=2, metavar=("MODE", "DIR"),
                    help="write the kernel-trace summary of the backward ('backward') or the "
                         "module with projections ('projections') of --workload from a "
                         "rocprofv3 --kernel-trace --stats output folder and exit")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("PMC_DIR", "TRACE_DIR"),
                    help="write the matrix-core busy summary of --workload from a rocprofv3 "
                         "--pmc MfmaUtil output folder and a --kernel-trace folder and exit")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="write the kernel-trace summary of --workload from a rocprofv3 "
                         "--kernel-trace --stats output folder and exit")
    args = ap.parse_args()
    if args.passes_summary:
        from efficient_attention_vision_amd import inputs
        mode, folder = args.passes_summary
        if mode not in PASS_NAMES:
            sys.exit(f"bench.py: --passes-summary takes one of {sorted(PASS_NAMES)}")
        write_passes_summary(inputs.WORKLOADS[args.workload], mode, folder)
        return
    if args.pmc_summary or args.trace_summary or args.mfma_summary:
        from efficient_attention_vision_amd import inputs
        wl = inputs.WORKLOADS[args.workload]
        if args.mfma_summary:
            write_mfma_summary(wl, *args.mfma_summary)
        if args.pmc_summary:
            write_counter_summary(wl, *args.pmc_summary)
        if args.trace_summary:
            write_trace_summary(wl, args.trace_summary)
        return
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
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
    if args.dtype and wl.dtype != "f32":
        import dataclasses
        wl = dataclasses.replace(wl, dtype=args.dtype)
    if args.projections:
        args.module = True
    if (args.module or args.backward) and args.layout != "bhnd":
        print("bench.py: --module takes the dense layout only", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[wl.dtype]
    shape = (wl.B, wl.H, wl.N, wl.d)
    set_bytes = algorithmic_bytes(wl)
    R = max(2, min(args.steps, math.ceil((1 << 30) / set_bytes)))
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    sets = []
    store = (wl.B, wl.N, wl.H, wl.d) if args.layout == "bnhd" else shape
    for _ in range(R):
        q, k, v = (torch.randn(store, generator=gen, device=dev, dtype=torch.float32)
                   .mul_(wl.sigma).to(dt) for _ in range(3))
        if args.layout == "bnhd":
            q, k, v = (t.transpose(1, 2) for t in (q, k, v))
        a = (torch.randn((wl.B, wl.H, wl.k, wl.d), generator=gen, device=dev).to(dt)
             if wl.supplied_agents else None)
        out = torch.empty_strided(q.shape, q.stride(), dtype=dt, device=dev)
        sets.append((q, k, v, a, out))
    need = _binding.agent_attn_workspace_bytes(wl.B, wl.H, wl.h, wl.w, wl.d, wl.s,
                                               0 if wl.dtype == "f32" else 1)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    mod = {}
    if args.module:   # module parameters, shared by the batch (same recipe as the tests)
        mod = {"bias_agg": torch.randn((wl.H, wl.k, wl.N), generator=gen, device=dev),
               "bias_bcast": torch.randn((wl.H, wl.N, wl.k), generator=gen, device=dev),
               "dwc_weight": torch.randn((wl.H * wl.d, 3, 3), generator=gen, device=dev) / 3,
               "dwc_bias": 0.5 * torch.randn((wl.H * wl.d,), generator=gen, device=dev)}

    C = wl.H * wl.d
    if args.projections:   # token features per set; weights (N(0, 1/C)) and biases shared
        xs = [torch.randn((wl.B, wl.N, C), generator=gen, device=dev).to(dt) for _ in range(R)]
        wqkv = (torch.randn((3 * C, C), generator=gen, device=dev) / math.sqrt(C)).to(dt)
        wout = (torch.randn((C, C), generator=gen, device=dev) / math.sqrt(C)).to(dt)
        bqkv = 0.1 * torch.randn((3 * C,), generator=gen, device=dev)
        bout = 0.1 * torch.randn((C,), generator=gen, device=dev)
        ys = [torch.empty_like(x) for x in xs[:2]]
        pws = torch.zeros(max(1, _binding.lib().agent_attn_module_workspace_bytes(
            wl.B, wl.H, wl.h, wl.w, wl.d, wl.s, {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype])),
            dtype=torch.uint8, device=dev)
    if args.backward:
        bws = torch.empty(max(1, _binding.agent_attn_backward_workspace_bytes(
            wl.B, wl.H, wl.h, wl.w, wl.d, wl.s, {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype])),
            dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, a, o = sets[i % R]
        if args.backward:   # the output buffer of the set serves as dO
            eav.agent_attn_backward(q, k, v, o, (wl.h, wl.w), wl.s, wl.scale, agents=a,
                                    workspace=bws)
        elif args.projections:
            eav.agent_attn_module_forward(xs[i % R], wqkv, (wl.h, wl.w), wl.s, wl.H, wl.scale,
                                          b_qkv=bqkv, w_out=wout, b_out=bout, agents=a,
                                          out=ys[i % 2], workspace=pws, **mod)
        elif args.module:
            eav.agent_attn_forward_module(q, k, v, (wl.h, wl.w), wl.s, wl.scale, agents=a, out=o,
                                          workspace=ws, **mod)
        else:
            eav.agent_attn_forward(q, k, v, (wl.h, wl.w), wl.s, wl.scale, agents=a, out=o,
                                   workspace=ws)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # eager launches, each bracketed by events on the launch stream: the
    # spread of single-launch latencies (event overhead included)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    eager_us = sorted(1e3 * a.elapsed_time(b) for a, b in evs)

    def pct(p):
        return eager_us[min(len(eager_us) - 1, int(p * len(eager_us)))]

    # graph of exactly K steps; the timed region is one replay of it, with
    # events recorded on the stream the kernels run on
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = 1e3 * (t1 - t0) / args.steps
    kernel_us = 1e3 * e0.elapsed_time(e1) / args.steps   # one launch per step

    tokens = wl.B * wl.H * wl.N
    value = tokens / (ms_per_step * 1e-3)
    abytes = algorithmic_bytes(wl)
    aflops = algorithmic_flops(wl)
    if args.module:   # + the two biases (read once, shared by the batch), + 9 MACs per output
        abytes += 2 * wl.H * wl.k * wl.N * 4
        aflops += 18 * wl.B * wl.H * wl.N * wl.d
    if args.backward:  # q, k, v, dO read and dq, dk, dv written; 8 + 16 products of N k d MACs
        abytes = abytes // 4 * 7
        aflops = aflops * 3
    if args.projections:   # x read and y written (q, k, v, o are intermediates), the
        # weights and the two biases; + 4 C MACs per token and output channel (projections)
        abytes = 2 * wl.B * wl.N * C * wl.es + 4 * C * C * wl.es + 2 * wl.H * wl.k * wl.N * 4
        aflops += 8 * wl.B * wl.N * C * C
    achieved_gbs = abytes / (kernel_us * 1e-6) / 1e9
    achieved_tflops = aflops / (kernel_us * 1e-6) / 1e12
    # counters were taken on the plain bf16 dense kernel: other variants report none
    plain = (not args.module and not args.backward and args.layout == "bhnd"
             and wl.dtype in ("bf16", "f32"))
    traffic = measured_traffic(wl.name) if plain else None
    # 16-bit tensors with up to 256 agents: token-tiled matrix-core passes, at
    # 24 k / 14 flop per byte; above the ridge (2.5 PFLOP/s over 8 TB/s, about
    # 180 agents) the matrix cores bound them; otherwise float32 products
    mfma_bwd = args.backward and wl.dtype != "f32" and wl.k <= 256
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bwd and aflops / abytes > ridge:
        roof = {"bound": "mfma", "achieved": achieved_tflops, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved_tflops / BF16_PEAK_TFLOPS, "traffic": traffic}
    elif mfma_bwd:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic}
    elif args.backward:   # float32 vector arithmetic (no matrix cores)
        roof = {"bound": "alu", "achieved": achieved_tflops, "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved_tflops / FP32_VECTOR_PEAK_TFLOPS,
                "traffic": traffic}
    elif wl.k >= 256:
        roof = {"bound": "mfma", "achieved": achieved_tflops, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved_tflops / BF16_PEAK_TFLOPS, "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic}
    line = {
        "metric": ("agent-attn bwd tokens/s (B*H*N/s)" if args.backward else
                   "agent-attn module fwd tokens/s (B*N*H/s), x -> y with projections"
                   if args.projections else
                   "agent-attn fwd tokens/s (B*H*N/s) + achieved HBM GB/s at N=3136,k=49 bf16"),
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
                   "supplied_agents": wl.supplied_agents, "rotating_sets": R,
                   "layout": "[B,N,H,d] storage" if args.layout == "bnhd" else "[B,H,N,d]",
                   **({"module_terms": ["agent biases B1, B2", "depth-wise 3x3 conv of V"]}
                      if args.module else {}),
                   **({"projections": ["x -> q, k, v (C -> 3C)", "o -> y (C -> C)"], "C": C}
                      if args.projections else {}),
                   **({"pass": "backward (dq, dk, dv)",
                       "backward_path": ("matrix-core token passes" if mfma_bwd
                                         else "float32 products")} if args.backward else {})},
        "roofline": roof,
        "kernel_us_per_launch": kernel_us,
        "eager_launch_us": {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9)},
        "achieved_hbm_gbs": achieved_gbs,
        "achieved_tflops": achieved_tflops,
        "algorithmic_bytes": abytes,
        "algorithmic_flops": aflops,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, args.cpu_seconds, module=args.module)
        cb.pop("seconds", None)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
