"""Benchmark of the fused attention forward on one MI355X.

A step is one attn_fwd call over one batch of the workload (all steps of the
path: validation, address folding, tile loads, QK^T, bias, mask, online
softmax, PV, epilogue).  Default workload: Swin-T stage-1 shifted-window
attention (8 images of 56x56 tokens, 7x7 windows, shift 3, 3 heads, d=32,
f16, table bias and region mask, image layout).  ``--config`` selects another
workload (C1, C2, C3, C3i, C4, C4h, C5s, C5x; C3i is C3 read from the
unpadded 64x64 token image in the image layout).

Inputs are resident in HBM before timing starts.  Several copies of the input
set rotate so that every launch reads data that is not in the 256 MB
Infinity Cache (at least 512 MB of distinct buffers in total).

Prints one JSON line with the throughput, a roofline record for the kernel
(algorithmic bytes or flops per launch over the mean launch duration measured
with HIP events on the launch stream) and the oracle's CPU throughput.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (and GB/s) per config, % of MI355X bf16 MFMA / HBM peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_MFMA_TFLOPS = 2500.0      # dense bf16/fp16 MFMA
PEAK_F32_TFLOPS = 157.3        # fp32 vector
RIDGE = PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed, so
    that a stored counter record stays valid across comment-only edits."""
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_dot_product_16_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_record(w):
    """HBM bytes per launch from the committed rocprofv3 counter record of this
    workload, if it was taken on the current kernel sources (else None)."""
    import glob

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{w.name}_traffic.json"))):
        with open(path) as f:
            rec = json.load(f)
        if rec.get("workload") == w.name and rec.get("kernel_source_hash") == kernel_source_hash():
            return rec.get("hbm_bytes_per_launch")
    return None


def device_clocks(dev: int) -> dict:
    """Peak engine and memory clocks (kHz) from the HIP runtime, or {}."""
    import ctypes

    # hipDeviceAttribute_t values of hipDeviceAttributeClockRate and
    # hipDeviceAttributeMemoryClockRate in hip_runtime_api.h (ROCm 7).
    attrs = {"peak_clock_khz": 5, "peak_memory_clock_khz": 60}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return {}
    out = {}
    for key, attr in attrs.items():
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(attr), ctypes.c_int(dev)) == 0:
            out[key] = v.value
    return out


def cpu_baseline(w, budget_s: float = 10.0):
    """Time the fp64 oracle on this host on a bounded sample of the workload."""
    import numpy as np

    import oracle
    from scaled_dot_product_16_amd import workloads as W

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    inp = W.make_inputs(w)
    arrs = {k: v.double().numpy() for k, v in inp.items()}
    if w.layout == "image":
        # Whole workload per repetition.
        flops_per_rep = w.flops
        sample = f"whole workload ({w.B} windows x {w.H} heads), repeated"
        run = lambda: oracle.run_workload(w, arrs)
    else:
        # A fixed set of (batch item, head) units, every query row of each.
        units = []
        rng = np.random.default_rng(7)
        cost_unit = 4 * w.Nq * w.Nk * w.d
        n_units = max(1, min(w.B * w.H, int(2e9 // cost_unit)))
        for _ in range(n_units):
            units.append((int(rng.integers(w.B)), int(rng.integers(w.H)), np.arange(w.Nq)))
        flops_per_rep = cost_unit * n_units
        sample = f"{n_units} (batch item, head) units, all query rows, repeated"
        run = lambda: oracle.run_workload(w, arrs, select=units)
    reps, t_total = 0, 0.0
    while reps < 1 or t_total < budget_s:
        t0 = time.perf_counter()
        run()
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": round(flops_per_rep * reps / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{sample} {reps}x, {t_total:.1f} s, numpy float64"}


def copy_calibration(torch, mib: int):
    """Plain device-to-device copies of a known size.  Under a counter run the
    per-dispatch FETCH_SIZE / WRITE_SIZE of these copies, divided by the bytes
    they must move (mib MiB each way), give the scale applied to the attention
    kernel's counters."""
    n = mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0").normal_()
    dst = [torch.empty_like(src) for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(5):
        dst[i % 2].copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "dispatches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="GPU time of untimed graph replays before the timed one (clock ramp-up)")
    ap.add_argument("--config", default="C2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches with per-launch events instead of a graph replay")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (reference dispatches "
                         "for scaling the HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return

    from scaled_dot_product_16_amd import binding
    from scaled_dot_product_16_amd import workloads as W

    w = W.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    binding.lib()
    inp = W.make_inputs(w)
    base = {k: v.to(dev) for k, v in inp.items()}
    set_bytes = sum(t.numel() * t.element_size() for t in base.values()) + \
        base["q"].numel() * base["q"].element_size()
    n_sets = max(1, math.ceil(512e6 / set_bytes))
    sets = []
    for i in range(n_sets):
        s = {k: (v.clone() if k in ("q", "k", "v") else v) for k, v in base.items()}
        s["out"] = torch.empty_like(base["q"])
        s["kw"] = W.device_args(w, s)
        sets.append(s)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = sets[i % n_sets]
        binding.fwd(s["q"], s["k"], s["v"], out=s["out"], **s["kw"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    if args.no_graph:
        # Eager launches with an event pair around each one.
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(K):
            ev[i][0].record(stream)
            step(i)
            ev[i][1].record(stream)
        t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        launch_ms = sorted(a.elapsed_time(b) for a, b in ev)
        mean_launch_ms = sum(launch_ms) / K
        median_launch_ms = launch_ms[K // 2]
        timing = "eager launches, HIP event pair per launch"
    else:
        # The K steps are captured once into a HIP graph (the library never
        # allocates or synchronises, so its launches capture as-is) and the
        # graph is replayed: back-to-back dispatches without host launch gaps.
        # The replayed result is checked against the eager one first.
        ref = sets[0]["out"].clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(sets[0]["out"], ref):
            raise RuntimeError("graph replay output differs from the eager output")
        # After an idle gap the clocks take some 10-20 ms of sustained work to
        # ramp up: untimed back-to-back replays (about --settle-ms of GPU
        # time, at most 30 of them: hundreds of replays of microsecond
        # kernels made the following timed replay noisier, not steadier) come
        # before the timed one, so it measures the steady state.
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        g.replay()
        w1.record(stream)
        torch.cuda.synchronize()
        n_settle = min(30, max(2, math.ceil(args.settle_ms / max(w0.elapsed_time(w1), 1e-3))))
        for _ in range(n_settle):
            g.replay()
        torch.cuda.synchronize()
        t_start.record(stream)
        g.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        mean_launch_ms = median_launch_ms = total_ms / K
        timing = (f"HIP graph of K launches, HIP events around one replay, after {n_settle + 1} "
                  f"untimed back-to-back replays that settle the clocks")
    ms_per_step = total_ms / K

    flops = w.flops
    nbytes = w.algorithmic_bytes
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    ai = flops / nbytes
    if w.dtype == W.F32:
        bound = "hbm" if ai < PEAK_F32_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "alu"
    else:
        bound = "hbm" if ai < RIDGE else "mfma"
    if bound == "hbm":
        achieved = nbytes / (mean_launch_ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    elif bound == "alu":
        achieved = flops / (mean_launch_ms * 1e-3) / 1e12
        peak, unit = PEAK_F32_TFLOPS, "TFLOP/s"
    else:
        achieved = flops / (mean_launch_ms * 1e-3) / 1e12
        peak, unit = PEAK_MFMA_TFLOPS, "TFLOP/s"

    cfg = {"workload": w.name, "batch_items": w.B, "heads": w.H, "q_tokens": w.Nq,
           "kv_tokens": w.Nk, "head_dim": w.d, "bias": w.bias, "mask": w.mask,
           "layout": w.layout}
    if w.window:
        cfg["image"] = f"{w.images}x{w.window[0]}x{w.window[1]}"
        cfg["window"] = f"{w.window[2]}x{w.window[3]}"
        cfg["shift"] = list(w.window[4:])
    if w.grid:
        cfg["grid"] = list(w.grid)

    props = torch.cuda.get_device_properties(dev)
    device = {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count, **device_clocks(dev.index or 0),
              "hip": torch.version.hip, "torch": torch.__version__,
              "peaks": {"hbm_GBs": PEAK_HBM_GBS, "bf16_fp16_mfma_TFLOPs": PEAK_MFMA_TFLOPS,
                        "fp32_TFLOPs": PEAK_F32_TFLOPS}}
    line = {
        "metric": METRIC,
        "value": round(tflops, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, N(0,0.02^2) tables)",
        "config": cfg,
        "gb_per_s": round(gbs, 2),
        "flops_per_step": flops,
        "algorithmic_bytes_per_step": nbytes,
        "rotating_input_sets": n_sets,
        "device": device,
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic_record(w),
            "kernel_mean_ms": round(mean_launch_ms, 6),
            "kernel_median_ms": round(median_launch_ms, 6),
            "timing": timing,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
