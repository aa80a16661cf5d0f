"""Benchmark of the gfx950 attention forward (one JSON line on stdout).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one attn_fwd call (the whole hot path) on the headline workload:
B=2, H=32, N=8192, d=128, non-causal, bf16 inputs already resident in device
memory. The metric is attention TFLOP/s = 4*B*H*N^2*d (halved for causal) /
kernel time, and its fraction of the MI355X dense bf16 matrix-core peak
(2500 TFLOP/s). The other workloads are timed too and reported under
"workloads" for context. The fp64 CPU oracle is timed on the host cores on a
bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The CPU baseline's BLAS threads: every core this process may run on, unless the
# environment already fixes the count (set before numpy or torch loads a BLAS).
AFFINITY_CORES = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(AFFINITY_CORES))

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "exact_attention_22_amd", "csrc")
KERNEL_SOURCES = ("attn_fwd_kernel.h", "attn_fwd.hip", "attn_fwd_launch.h", "attn_fwd_launch_impl.h",
                  "attn_fwd_d128_full.hip", "exp2_poly.h")

# HBM bytes per launch of the headline kernel from two rocprofv3 --pmc runs
# (FETCH_SIZE and WRITE_SIZE, KiB per dispatch), each scaled by what the same
# counter reads for a 256 MiB device copy (FETCH x2.0, WRITE x1.0); see
# profiles/attn_fwd_headline_counters.md. Valid only for the kernel sources
# with this SHA-256; any change to them reports traffic as null.
TRAFFIC = {"sources_sha256": "f50e50ad9d246464e4dc8cb1d9eefc27e7ed10a75e475fec4b60e5a753dec171",
           "fetch_kib": 196768.2, "write_kib": 133120.0, "fetch_scale": 2.0, "write_scale": 1.0}


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(workload_name: str):
    if workload_name != "headline" or kernel_sources_sha256() != TRAFFIC["sources_sha256"]:
        return None
    return int((TRAFFIC["fetch_kib"] * TRAFFIC["fetch_scale"] + TRAFFIC["write_kib"] * TRAFFIC["write_scale"]) * 1024)


def describe(w) -> str:
    from exact_attention_22_amd import inputs
    if isinstance(w, inputs.VarlenWorkload):
        L = w.lengths
        return (f"{w.B} packed sequences of {min(L)}..{max(L)} tokens (total {sum(L)}) H={w.H} Hkv={w.Hkv} "
                f"d={w.d}")
    return f"B={w.B} H={w.H} Hkv={w.kv_heads} N={w.N} d={w.d}"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-others", action="store_true",
                    help="time only the K headline steps (no other workloads, no sampled timing)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU oracle time")
    ap.add_argument("--mode", choices=("forward", "backward", "splitkv", "fp8"), default="forward",
                    help="backward / splitkv: time only that path on --workload (a dense workload) and print "
                         "one short JSON line (for profiling); forward: the benchmark line")
    ap.add_argument("--exp2-poly-eighths", type=int, default=0, choices=(0, 4, 8),
                    help="forward timing with this many of every 8 exponentials on the polynomial (default 0)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (calibrates profiler byte counters)")
    return ap.parse_args()


def workload_call(w, **kw):
    """Device-resident inputs and outputs of a workload and a function that runs one
    launch of the attention forward on them (dense or packed variable-length)."""
    import torch

    from exact_attention_22_amd import binding, inputs

    dev = torch.device("cuda:0")
    if isinstance(w, inputs.VarlenWorkload):
        q, k, v, cu = (t.to(dev) for t in w.inputs())
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        max_seqlen = max(w.lengths)

        def call():
            binding.attention_varlen(q, k, v, cu, max_seqlen, causal=w.causal, scale=w.scale, out=o, lse=lse, **kw)
    else:
        q, k, v = (t.to(dev) for t in inputs.workload_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def call():
            binding.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, **kw)
    return call


def time_workload(w, steps, warmup, **kw):
    """Average kernel time (ms) over `steps` launches, bracketed by device syncs,
    measured with HIP events on the stream the kernel is launched on."""
    import torch

    dev = torch.device("cuda:0")
    call = workload_call(w, **kw)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del call
    torch.cuda.empty_cache()
    return ms


def time_backward(w, steps, warmup):
    """Average time (ms) of one attn_bwd call (dq and dk/dv kernels) on a dense
    workload's shape, with O and LSE from one forward pass; dO drawn N(0,1)."""
    import torch

    from exact_attention_22_amd import binding, inputs

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inputs.workload_inputs(w))
    do = inputs.draw(w.B, w.H, w.N, w.d, seed=w.seed + 7919)[0].to(dev)
    o, lse = binding.attention(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)

    def call():
        binding.attention_backward(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                                   delta=delta)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del q, k, v, do, o, lse, dq, dk, dv, delta
    torch.cuda.empty_cache()
    return ms


def time_split(w, steps, warmup):
    """Average time (ms) of attn_fwd_splitkv (automatic split count, partial and merge
    kernels) on a dense workload, workspace allocated once beforehand."""
    import torch

    from exact_attention_22_amd import binding, inputs

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in inputs.workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.splitkv_workspace_size(w.B, w.H, w.N, w.d, 0), dtype=torch.uint8, device=dev)

    def call():
        binding.attention_splitkv(q, k, v, causal=w.causal, scale=w.scale, n_splits=0, out=o, lse=lse, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return ms


def time_backward_varlen(w, steps, warmup):
    """Average time (ms) of one attn_bwd_varlen call on a packed workload (O and LSE from one
    attn_fwd_varlen pass; dO drawn N(0,1))."""
    import torch

    from exact_attention_22_amd import binding

    dev = torch.device("cuda:0")
    q, k, v, cu = (t.to(dev) for t in w.inputs())
    g = torch.Generator(device="cpu").manual_seed(w.seed + 7919)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
    mx = max(w.lengths)
    o, lse = binding.attention_varlen(q, k, v, cu, max_seqlen=mx, causal=w.causal, scale=w.scale)

    def call():
        binding.attention_backward_varlen(q, k, v, o, lse, do, cu, max_seqlen=mx, causal=w.causal, scale=w.scale)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del q, k, v, cu, do, o, lse
    torch.cuda.empty_cache()
    return ms


def time_fp8(w, steps, warmup):
    """Average time (ms) of attn_fwd_fp8 on a dense workload's shape: the same N(0,1)
    draws quantised to e4m3 with per-tensor scales, V transposed."""
    import torch

    from exact_attention_22_amd import binding, inputs

    dev = torch.device("cuda:0")
    q8, k8, vt8, sc = inputs.draw_fp8(w.B, w.H, w.N, w.d, seed=w.seed, drift=w.drift)
    q8, k8, vt8 = q8.to(dev), k8.to(dev), vt8.to(dev)
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def call():
        binding.attention_fp8(q8, k8, vt8, sc, causal=w.causal, scale=w.scale, out=o, lse=lse)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del q8, k8, vt8, o, lse
    torch.cuda.empty_cache()
    return ms


class ClockSampler(threading.Thread):
    """Reads the GPU's current SCLK with rocm-smi (a child process) about every 0.3 s while
    the timed samples run; values in MHz, empty if rocm-smi is absent or prints no clock."""

    def __init__(self):
        super().__init__(daemon=True)
        self.mhz = []
        self.done = threading.Event()

    def run(self):
        while not self.done.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            self.mhz += [int(m.group(1)) for m in re.finditer(r"sclk[^\n]*?\((\d+)\s*mhz\)", out, re.I)]
            self.done.wait(0.3)

    def summary(self):
        self.done.set()
        self.join(timeout=15)
        if not self.mhz:
            return None
        v = sorted(self.mhz)
        return {"n": len(v), "median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1]}


def time_samples(w, n_samples=20, min_ms=50.0):
    """n_samples timed batches of back-to-back launches, each at least min_ms long;
    per-launch median and min (ms)."""
    import torch

    dev = torch.device("cuda:0")
    call = workload_call(w)
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def batch(n):
        start.record(stream)
        for _ in range(n):
            call()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    one = batch(3) / 3
    per_batch = max(1, int(math.ceil(min_ms / max(one, 1e-3))))
    ms = sorted(batch(per_batch) / per_batch for _ in range(n_samples))
    del call
    torch.cuda.empty_cache()
    return {"n": n_samples, "launches_each": per_batch, "median_ms": round(ms[len(ms) // 2], 4),
            "min_ms": round(ms[0], 4)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, target_s):
    """Time the fp64 oracle (as it stands) on a bounded sample: whole heads of the
    workload, as many as fit the target time; returned in TFLOP/s of the metric."""
    import numpy as np  # noqa: F401  (loads the BLAS whose threads are counted below)
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [0])
    except Exception:  # threadpoolctl absent
        blas = 0
    threads = blas or int(os.environ.get("OPENBLAS_NUM_THREADS") or AFFINITY_CORES)
    import oracle
    from exact_attention_22_amd import inputs

    if isinstance(w, inputs.VarlenWorkload):  # whole heads of the packed batch
        units = w.H

        def run(n, seed):
            q, k, v, cu = inputs.draw_varlen(w.lengths, n, n, w.d, seed=seed)
            t0 = time.perf_counter()
            oracle.attention_varlen(q, k, v, cu, w.causal, w.scale)
            return time.perf_counter() - t0
    else:
        units = w.B * w.H

        def run(n, seed):
            q, k, v = inputs.draw(1, n, w.N, w.d, seed=seed, drift=w.drift)
            t0 = time.perf_counter()
            oracle.attention(q, k, v, w.causal, w.scale)
            return time.perf_counter() - t0

    one = run(1, w.seed)
    heads = max(1, min(units, int(target_s / max(one, 1e-3))))
    dt = run(heads, w.seed + 1)
    flops = w.flops / units * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {units} heads of {w.name} (full rows), {dt:.1f} s fp64 numpy",
            "seconds": round(dt, 2), "cpu_model": cpu_model(), "blas_threads": int(threads),
            "host_cpus": os.cpu_count(), "affinity_cpus": AFFINITY_CORES,
            "thread_env": {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")},
            "full_workload_seconds_extrapolated": round(dt * units / heads, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by heads with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch

    from exact_attention_22_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    binding.lib()  # fail loudly if the HIP library is missing
    by_name = dict(inputs.BY_NAME, **{inputs.VARLEN.name: inputs.VARLEN, inputs.LOWOCC.name: inputs.LOWOCC})
    w = by_name[args.workload]

    is_varlen = isinstance(w, inputs.VarlenWorkload)
    if args.mode != "forward":
        if is_varlen:
            print("--mode backward/splitkv needs a dense workload", file=sys.stderr)
            sys.exit(2)
        if args.mode == "backward":
            ms = time_backward(w, args.steps, args.warmup)
            flops = 2.5 * w.flops  # five N^2 d products against the forward's two
        elif args.mode == "fp8":
            ms = time_fp8(w, args.steps, args.warmup)
            flops = w.flops
            if args.copy_mib:  # calibration copy for the profiler's byte counters
                src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda:0")
                torch.empty_like(src).copy_(src)
                torch.cuda.synchronize()
        else:
            ms = time_split(w, args.steps, args.warmup)
            flops = w.flops
        print(json.dumps({"mode": args.mode, "workload": f"{w.name}: {describe(w)} causal={w.causal}",
                          "steps": args.steps, "ms_per_step": round(ms, 4),
                          "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}), flush=True)
        return
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_workload(w, args.steps, args.warmup, poly_eighths=args.exp2_poly_eighths)
    wall = time.perf_counter() - t0
    tflops = w.flops / (ms * 1e-3) / 1e12
    samples = None
    if not args.no_others:  # 20 batches of >= 50 ms of back-to-back launches: median and min
        clock = ClockSampler()
        clock.start()
        samples = time_samples(w)
        samples["sclk"] = clock.summary()
        samples["median_tflops"] = round(w.flops / (samples["median_ms"] * 1e-3) / 1e12, 1)
        samples["max_tflops"] = round(w.flops / (samples["min_ms"] * 1e-3) / 1e12, 1)

    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    others = {}
    if not args.no_others:
        for o in inputs.WORKLOADS + [inputs.VARLEN]:
            if o.name == w.name:
                continue
            oms = time_workload(o, max(5, args.steps // 2), max(3, args.warmup // 2))
            ot = o.flops / (oms * 1e-3) / 1e12
            others[o.name] = {"ms": round(oms, 4), "tflops": round(ot, 1),
                              "frac_peak": round(ot / PEAK_BF16_TFLOPS, 4), "causal": o.causal,
                              "shape": describe(o)}

    backward = {}
    if not args.no_others:  # backward pass (2.5x the forward flops: five N^2 d products)
        for name in ("headline", "causal2k", "long32k"):
            o = inputs.BY_NAME[name]
            bms = time_backward(o, max(5, args.steps // 5), 3)
            bt = 2.5 * o.flops / (bms * 1e-3) / 1e12
            backward[name] = {"ms": round(bms, 4), "tflops": round(bt, 1), "frac_peak": round(bt / PEAK_BF16_TFLOPS, 4),
                              "causal": o.causal, "shape": describe(o)}
        vw = inputs.VARLEN
        bms = time_backward_varlen(vw, max(5, args.steps // 5), 3)
        bt = 2.5 * vw.flops / (bms * 1e-3) / 1e12
        backward[vw.name] = {"ms": round(bms, 4), "tflops": round(bt, 1), "frac_peak": round(bt / PEAK_BF16_TFLOPS, 4),
                             "causal": vw.causal, "shape": describe(vw)}

    splitkv = {}
    if not args.no_others:  # split keys on shapes with fewer query tiles than compute units
        for sw in (inputs.LOWOCC, inputs.Workload("lowocc_causal32k", 1, 4, 32768, 128, True, False, 1104)):
            plain = time_workload(sw, 10, 3)
            split = time_split(sw, 10, 3)
            splitkv[sw.name] = {"shape": describe(sw), "causal": sw.causal, "ms_plain": round(plain, 4),
                                "ms_split": round(split, 4),
                                "tflops_plain": round(sw.flops / (plain * 1e-3) / 1e12, 1),
                                "tflops_split": round(sw.flops / (split * 1e-3) / 1e12, 1)}

    fp8 = {}
    if not args.no_others:  # FP8 (e4m3) forward, against the dense fp8 matrix-core peak
        for name in ("headline", "causal2k", "long32k", "drift8k"):
            o = inputs.BY_NAME[name]
            fms = time_fp8(o, max(5, args.steps // 2), 3)
            ft = o.flops / (fms * 1e-3) / 1e12
            fp8[name] = {"ms": round(fms, 4), "tflops": round(ft, 1), "frac_peak_fp8": round(ft / PEAK_FP8_TFLOPS, 4),
                         "causal": o.causal, "shape": describe(o)}

    line = {
        "metric": "attention fwd TFLOP/s (bf16, causal & non-causal) and % of MI355X MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {describe(w)} causal={w.causal} bf16 N(0,1) seed {w.seed}",
                   "B": w.B, "H": w.H, "Hkv": w.Hkv if is_varlen else w.kv_heads,
                   "N": max(w.lengths) if is_varlen else w.N, "d": w.d, "causal": w.causal,
                   "exp2_poly_eighths": args.exp2_poly_eighths},
        "frac_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_bytes(w.name) if args.exp2_poly_eighths == 0 else None},
        "timed_wall_s": round(wall, 2),
        "samples": samples,
        "workloads": others,
        "backward": backward,
        "splitkv": splitkv,
        "fp8": fp8,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        line["gpu_speedup_vs_cpu_baseline"] = round(tflops / line["cpu_baseline"]["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
