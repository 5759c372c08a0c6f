#!/usr/bin/env python3
"""Benchmark of the gfx950 dense attention forward (bf16, head_dim 128, non-causal).

One step = one attention forward over the whole workload (one kernel
launch, every (b, h, 128-row tile) of the batch). Inputs are seeded
synthetic tensors already resident in HBM when timing starts. Prints one
JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak (published)
METRIC = "attn fwd TFLOP/s (bf16, hd128, non-causal) S=4K/8K/16K; % MFMA peak"
HEADLINE = "s16k_outliers"
ALSO = ["s4k", "s8k_peaked", "s16k_outliers"]
KERNEL_SOURCES = [ROOT / "dense_attention_forward_amd" / "csrc" / n
                  for n in ("attn_fwd_kernel.hip", "attn_fwd_abi.cpp", "attn_fwd_launch.h")]


def kernel_digest() -> str:
    """Hash of the kernel sources' code: // comments removed and whitespace
    collapsed, so edits to comments or layout keep the measured counters
    valid while any code change invalidates them."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        code = re.sub(r"//[^\n]*", "", p.read_text())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    f = ROOT / "profiles" / f"attn_fwd_traffic_{workload}.txt"
    if not f.exists():
        return None
    text = f.read_text()
    m_sha = re.search(r"^kernel_sources_sha256_16:\s*(\w+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != kernel_digest():
        return None
    return float(m_b.group(1))


def time_workload(daf, torch, w, steps: int, warmup: int, min_warm_s: float = 0.0):
    """Times `steps` launches after `warmup` untimed ones (and, with
    min_warm_s, more untimed ones until that much wall time has passed: the
    GPU idles while the inputs are drawn on the host, and its clock takes a
    while to come back up)."""
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        daf.forward(q, k, v, w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < min_warm_s:
        for _ in range(10):
            daf.forward(q, k, v, w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)  # the kernels are enqueued on this stream
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        daf.forward(q, k, v, w.scale, out=o, lse=lse)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    ok = bool(torch.isfinite(o).all().item() and torch.isfinite(lse).all().item())
    del q, k, v, o, lse
    return ms, wall, ok


def sustained_mfma(daf, torch, reps: int = 5, iters: int = 2000):
    """Rate of a pure v_mfma_f32_16x16x32_bf16 stream (no memory in the loop;
    the instruction of the eight-wave kernel) on N(0,1) bf16 operands, the
    workloads' distribution, 8 workgroups of 4 waves per CU. Under sustained
    MFMA load the clock is set by power, which depends on operand toggling,
    so this is what the matrix cores sustain on such data; the published
    peak assumes the top clock."""
    dev = torch.device("cuda", 0)
    wgs = torch.cuda.get_device_properties(dev).multi_processor_count * 8
    gen = torch.Generator(device=dev).manual_seed(7)
    operands = torch.randn(wgs * 256 * 64, generator=gen, device=dev).to(torch.bfloat16)
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    daf.mfma_rate(operands, sink, wgs, 200)
    torch.cuda.synchronize()
    rates = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        flops = daf.mfma_rate(operands, sink, wgs, iters)
        end.record()
        torch.cuda.synchronize()
        rates.append(flops / (start.elapsed_time(end) * 1e-3) / 1e12)
    rates.sort()
    return {"value": round(rates[-1], 1), "median": round(rates[len(rates) // 2], 1), "unit": "TFLOP/s",
            "operands": "bf16 N(0,1)", "launches": reps,
            "kernel": "attn_mfma_rate: v_mfma_f32_16x16x32_bf16 stream from registers, 8 accumulators "
                      "in VGPRs, 8 workgroups of 4 waves per CU"}


def cpu_baseline(w, max_heads: int):
    """The fp64 oracle, untuned, on the first heads of the same workload."""
    import torch

    import oracle
    threads = len(os.sched_getaffinity(0))
    torch.set_num_threads(threads)
    q, k, v = workloads.make_inputs(w)
    nh = max(1, min(max_heads, w.H))
    qs, ks, vs = (t[:1, :nh].contiguous() for t in (q, k, v))
    t0 = time.perf_counter()
    oracle.attention(qs, ks, vs, w.scale)
    dt = time.perf_counter() - t0
    flops = 4 * nh * w.S * w.S * w.D
    cpu_model = ""
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"batch 0, heads 0..{nh - 1} of {w.name} (all {w.S} query rows each), "
                      f"fp64 two-pass oracle, {dt:.1f} s wall",
            "seconds": dt, "cpu": cpu_model or platform.processor(), "os_cpu_count": os.cpu_count()}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=HEADLINE, choices=[w.name for w in workloads.WORKLOADS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip timing the pure MFMA stream (the sustained matrix-core rate)")
    ap.add_argument("--no-also", action="store_true", help="skip the other sequence lengths")
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads in the CPU-baseline sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "reference reading for the HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the (b, h) work items are independent, so more GPUs "
              "would each run this same kernel on a share of the heads; no multi-GPU path is built.",
              file=sys.stderr)
        return 2

    import torch

    import dense_attention_forward_amd as daf
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    daf.lib()

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20)
        x = torch.ones(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)
        return 0

    w = workloads.get(args.workload)
    ms, wall, ok = time_workload(daf, torch, w, args.steps, args.warmup)
    tflops = w.flops / (ms * 1e-3) / 1e12
    per = {}
    if not args.no_also:
        for name in ALSO:
            if name == w.name:
                per[name] = {"tflops": round(tflops, 1), "ms": round(ms, 4)}
                continue
            wx = workloads.get(name)
            msx, _, okx = time_workload(daf, torch, wx, max(5, args.steps), 3, min_warm_s=0.3)
            ok = ok and okx
            per[name] = {"tflops": round(wx.flops / (msx * 1e-3) / 1e12, 1), "ms": round(msx, 4)}

    traffic = measured_traffic(w.name)
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": False,
                   "flops_per_step": w.flops, "seed": w.seed},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "per_workload": per,
        "outputs_finite": ok,
        "kernel_sources_sha256_16": kernel_digest(),
    }
    if not args.no_mfma_ceiling:
        sus = sustained_mfma(daf, torch)
        sus["frac_achieved"] = round(tflops / sus["value"], 4)
        line["mfma_sustained"] = sus
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_heads)
    print(json.dumps(line), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
