"""Benchmark of the fused attention forward on one MI355X.

A step is one attn_fwd call over one batch of the workload (all steps of the
path: validation, address folding, tile loads, QK^T, bias, mask, online
softmax, PV, epilogue).  Headline workload: Swin-T stage-1 shifted-window
attention (8 images of 56x56 tokens, 7x7 windows, shift 3, 3 heads, d=32,
f16, table bias and region mask, image layout).  ``--config`` selects another
headline (C1, C2, C3, C3i, C4, C4h, C5s, C5x; C3i is C3 read from the
unpadded 64x64 token image in the image layout).  Every other workload is
timed in the same run and reported under ``workloads`` (``--extra`` picks
them, ``--extra none`` skips them).

Inputs are resident in HBM before timing starts.  Several copies of the input
set rotate so that every launch reads data that is not in the 256 MB
Infinity Cache (at least 512 MB of distinct buffers in total).

Timing: the K steps are captured into a HIP graph; a second graph of
back-to-back launches (at least --settle-ms of GPU time) is queued first and
the timed graph right behind it, so the clocks have ramped up and the GPU
never idles before the timed launches; HIP events on the launch stream
bracket exactly the K timed steps, with device synchronisations before the
settle work and after the timed replay.

Prints one JSON line: the headline's throughput, its roofline record (bytes
or flops per launch over the mean launch duration), its max-abs error
against the fp64 oracle, the oracle's CPU throughput (process pool on the
host cores), a plain device copy of the headline's bytes measured the same
way (the copy floor), and one record per extra workload.
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
ALL = ["C1", "C2", "C3", "C3i", "C4", "C4h", "C5s", "C5x"]
# The Swin-T and SD workloads with q, k, v as 8-bit E4M3 codes (f16 compute).
LOW_PRECISION = ["C2f8", "C5sf8", "C5xf8"]
# Backward passes (attn_bwd) of Swin-T, SAM-B windowed and global, and SD
# self-attention: the workload key with a trailing "b".
BACKWARD = ["C2b", "C3b", "C4b", "C5sb"]
TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 2e-2}


# Sources that only hold the backward kernels, their plan, launchers and
# entry points; the forward kernels' counter records do not depend on them.
BACKWARD_ONLY_SOURCES = ("attn_bwd.h", "attn_bwd_launch.h", "attn_plan_bwd.h", "attn_noalloc.hip")


def kernel_source_hash() -> str:
    """Hash of the sources the forward kernels are built from, with comments
    and blank space removed, so that a stored counter record stays valid
    across comment-only edits and changes confined to the backward."""
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_dot_product_16_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name in BACKWARD_ONLY_SOURCES:
            continue
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


def sample_units(w, limit: int):
    """Up to ``limit`` units of the workload, spread evenly (first and last
    included)."""
    from oracle import pool

    units = pool.units_of(w)
    if len(units) <= limit:
        return units
    idx = sorted({round(i * (len(units) - 1) / (limit - 1)) for i in range(limit)})
    return [units[i] for i in idx]


def oracle_error(w, inp: dict, out, limit: int):
    """Max-abs error of the GPU output against the fp64 oracle on a sample of
    units (every output row of each), oracle units spread over the pool."""
    from oracle import pool

    units = sample_units(w, limit)
    with pool.UnitPool(dict(inp, out=out.detach().to("cpu")), pool.spec_of(w)) as P:
        res = P.compare(units)
    kind = "(image, head)" if w.layout == "image" else "(batch item, head)"
    return {"max_abs_err": max(r["err"] for r in res), "tol": TOL[w.dtype],
            "err_sample": f"{len(units)} of {len(pool.units_of(w))} {kind} units, every output row"}


def cpu_baseline(w, inp: dict, budget_s: float):
    """The fp64 oracle on this host's cores (one process per core, single-
    threaded BLAS), on a bounded sample of the workload's units."""
    from oracle import pool

    units = pool.units_of(w)
    unit_flops = w.flops // len(units)
    with pool.UnitPool(inp, pool.spec_of(w)) as P:
        n = P.workers
        # Size the sample from one round of one unit per worker.
        t1 = P.time_units(units[:n])
        per_round = max(t1, 1e-3)
        rounds = max(1, int(budget_s / per_round))
        sample = [units[i % len(units)] for i in range(rounds * n)]
        t = P.time_units(sample)
    kind = "(image, head)" if w.layout == "image" else "(batch item, head)"
    return {"value": round(unit_flops * len(sample) / t / 1e12, 6), "unit": "TFLOP/s", "cores": n,
            "kind": "oracle",
            "sample": f"{len(sample)} {kind} units of the workload (its {len(units)} units cycled), "
                      f"every output row, {t:.1f} s on a pool of {n} processes with single-threaded "
                      f"BLAS, numpy float64"}


def roofline_of(w, mean_ms: float, timing: str):
    flops, nbytes = w.flops, w.algorithmic_bytes
    ai = flops / nbytes
    if w.dtype == "f32":
        bound = "hbm" if ai < PEAK_F32_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "alu"
    else:
        bound = "hbm" if ai < RIDGE else "mfma"
    if bound == "hbm":
        achieved, peak, unit = nbytes / (mean_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    elif bound == "alu":
        achieved, peak, unit = flops / (mean_ms * 1e-3) / 1e12, PEAK_F32_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = flops / (mean_ms * 1e-3) / 1e12, PEAK_MFMA_TFLOPS, "TFLOP/s"
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_record(w),
            "kernel_mean_ms": round(mean_ms, 6), "timing": timing}


def config_of(w):
    cfg = {"workload": w.name, "batch_items": w.B, "heads": w.H, "q_tokens": w.Nq,
           "kv_tokens": w.Nk, "head_dim": w.d, "bias": w.bias, "mask": w.mask,
           "layout": w.layout}
    if w.window:
        cfg["image"] = f"{w.images}x{w.window[0]}x{w.window[1]}"
        cfg["window"] = f"{w.window[2]}x{w.window[3]}"
        cfg["shift"] = list(w.window[4:])
    if w.grid:
        cfg["grid"] = list(w.grid)
    if w.qkv != "same":
        cfg["qkv"] = f"{w.qkv} codes, one scale per tensor; {w.dtype} compute and output"
    return cfg


def timed_graph(torch, stream, step, K: int, settle_ms: float):
    """Capture K launches of ``step(i)`` into a graph, size a settle graph of
    about ``settle_ms`` of GPU time from one timed replay of it, then queue
    the settle graph and the timed one right behind it, between two events;
    return the timed milliseconds, a note and the graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            step(i)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    est_ms = t0.elapsed_time(t1) / K
    n_settle = max(2 * K, min(20000, math.ceil(settle_ms / max(est_ms, 1e-4))))
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gs):
        for i in range(n_settle):
            step(i)
    torch.cuda.synchronize()
    gs.replay()
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    del gs
    note = (f"HIP graph of K launches queued directly behind a graph of {n_settle} untimed "
            f"back-to-back launches (about {settle_ms:.0f} ms of clock settling, no idle gap); "
            f"HIP events around the K")
    return t0.elapsed_time(t1), note, g


def run_workload(torch, W, binding, w, K: int, warmup: int, settle_ms: float, no_graph: bool,
                 check_units: int, fwd_kw=None):
    """Time workload ``w``: rotating input sets, eager warmup, oracle check of
    the first output, then the graph-timed K steps.  ``fwd_kw``: extra
    arguments of the call (e.g. window_heads)."""
    dev = torch.device("cuda:0")
    inp = W.make_inputs(w)
    base = {k: v.to(dev) for k, v in inp.items()}
    out_dtype = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    set_bytes = sum(t.numel() * t.element_size() for t in base.values()) + \
        base["q"].numel() * w.bytes_per_elem()
    n_sets = max(1, math.ceil(512e6 / set_bytes))
    sets = []
    for i in range(n_sets):
        s = {k: (v.clone() if k in ("q", "k", "v") else v) for k, v in base.items()}
        s["out"] = torch.empty(base["q"].shape, dtype=out_dtype, device=dev)
        s["kw"] = dict(W.device_args(w, s), **(fwd_kw or {}))
        sets.append(s)
    del base
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = sets[i % n_sets]
        binding.fwd(s["q"], s["k"], s["v"], out=s["out"], **s["kw"])

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    rec = {}
    if check_units:
        rec.update(oracle_error(w, inp, sets[0]["out"], check_units))
    if no_graph:
        # Eager launches with an event pair around each one (profiler runs).
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            ev[i][0].record(stream)
            step(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        total_ms = sum(a.elapsed_time(b) for a, b in ev)
        note = "eager launches, HIP event pair per launch"
    else:
        ref = sets[0]["out"].clone()
        total_ms, note, g = timed_graph(torch, stream, step, K, settle_ms)
        # A replay rewrites set 0's output from set 0's inputs: it must equal
        # the eager result.
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(sets[0]["out"], ref):
            raise RuntimeError(f"{w.key}: graph replay output differs from the eager output")
        del g
    ms = total_ms / K
    rec.update({"ms_per_step": round(ms, 6), "tflops": round(w.flops / (ms * 1e-3) / 1e12, 4),
                "gb_per_s": round(w.algorithmic_bytes / (ms * 1e-3) / 1e9, 2),
                "flops_per_step": w.flops, "algorithmic_bytes_per_step": w.algorithmic_bytes,
                "rotating_input_sets": n_sets, "roofline": roofline_of(w, ms, note)})
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, inp


def run_backward(torch, W, binding, w, K: int, warmup: int, settle_ms: float, check_units: int):
    """Time the backward pass of workload ``w`` (attn_bwd_opt: dQ, dK, dV
    and the table gradients, given the forward's O and log-sum-exp as a
    training step has them), like run_workload.  Algorithmic
    work: the five products S, dP, dV, dK, dQ (10*B*H*Nq*Nk*d flops); bytes:
    Q, K, V, dO read and dQ, dK, dV written (plus the table and its
    gradient)."""
    import numpy as np

    import oracle

    dev = torch.device("cuda:0")
    inp = W.make_inputs(w)
    inp["dout"] = W.to_dtype(W.normal(w.q_shape, w.cfg_id, 7, 1.0), w.dtype)
    base = {k: v.to(dev) for k, v in inp.items()}
    per_set = 8 * base["q"].numel() * base["q"].element_size()
    n_sets = max(1, math.ceil(512e6 / per_set))
    sets = []
    for i in range(n_sets):
        s = {k: (v.clone() if k in ("q", "k", "v", "dout") else v) for k, v in base.items()}
        s["kw"] = W.device_args(w, s)
        # The forward's output and log-sum-exp, as a training step has them
        # (computed here, outside the timed region).
        s["lse"] = torch.empty(tuple(s["q"].shape[:3]), dtype=torch.float32, device=dev)
        s["out"] = binding.fwd(s["q"], s["k"], s["v"], lse=s["lse"], **s["kw"])
        s["dq"], s["dk"], s["dv"] = (torch.empty_like(s["q"]) for _ in range(3))
        s["dtable"] = (torch.empty(base["table"].shape, dtype=torch.float32, device=dev)
                       if w.bias == "table" else
                       torch.empty(base["rh"].shape[0] + base["rw"].shape[0], w.d, dtype=torch.float32,
                                   device=dev)
                       if w.bias == "relpos" else None)
        sets.append(s)
    # One workspace, reused by every launch (they run one after another).
    s0 = sets[0]
    binding.bwd(s0["q"], s0["k"], s0["v"], s0["dout"], dq=s0["dq"], dk=s0["dk"], dv=s0["dv"],
                dtable=s0["dtable"], out=s0["out"], lse=s0["lse"], **s0["kw"])
    import ctypes
    need = ctypes.c_size_t(0)
    qc, kc, vc, bd, md, oc, dt, keep = binding._marshal(s0["q"], s0["k"], s0["v"], s0["dout"],
                                                        s0["kw"].get("bias"), s0["kw"].get("mask"),
                                                        w.layout, s0["kw"].get("window"))
    binding.lib().attn_bwd_workspace_size(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc),
                                          ctypes.byref(oc), ctypes.byref(bd), ctypes.byref(md), dt,
                                          ctypes.byref(need))
    ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=dev)
    del keep
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = sets[i % n_sets]
        binding.bwd(s["q"], s["k"], s["v"], s["dout"], dq=s["dq"], dk=s["dk"], dv=s["dv"],
                    dtable=s["dtable"], workspace=ws, out=s["out"], lse=s["lse"], **s["kw"])

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    rec = {}
    if check_units:
        # Oracle gradients: the whole workload in the image layout or with a
        # table bias, else the first and last (batch item, head) units (no
        # bias or the relative position: each unit's dQ, dK, dV depend on its
        # own slice and the shared tables only; the table gradients, which
        # sum over all units, are checked at reduced sizes by the tests).
        arrs = {k: v.double().numpy() for k, v in inp.items()}
        got = [sets[0][k].detach().double().cpu().numpy() for k in ("dq", "dk", "dv")]
        errs = []
        if w.layout == "image" or w.bias == "table":
            ref = oracle.run_workload_backward(w, arrs)
            errs = [float(np.max(np.abs(g - ref[k]))) for g, k in zip(got, ("dq", "dk", "dv"))]
            sample = "whole workload"
            if w.bias == "table":
                errs.append(float(np.max(np.abs(sets[0]["dtable"].double().cpu().numpy() - ref["dtable"]))))
        else:
            bias = (oracle.Bias("relpos", grid=w.grid, rh=arrs["rh"], rw=arrs["rw"])
                    if w.bias == "relpos" else None)
            for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
                sl = {k: v[b:b + 1, h:h + 1] for k, v in arrs.items() if k in ("q", "k", "v", "dout")}
                ref = oracle.attention_backward(sl["q"], sl["k"], sl["v"], sl["dout"], bias)
                errs += [float(np.max(np.abs(g[b, h] - ref[k][0, 0]))) for g, k in zip(got, ("dq", "dk", "dv"))]
            sample = "2 (batch item, head) units, every row"
        rec.update({"max_abs_err": max(errs), "err_sample": sample})
    ref_out = sets[0]["dq"].clone()
    total_ms, note, g = timed_graph(torch, stream, step, K, settle_ms)
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(sets[0]["dq"], ref_out):
        raise RuntimeError(f"{w.key} backward: graph replay output differs from the eager output")
    del g
    ms = total_ms / K
    flops = 10 * w.B * w.H * w.Nq * w.Nk * w.d
    e = w.bytes_per_elem()
    nbytes = 7 * int(np.prod(w.q_shape)) * e
    if w.bias == "table":
        nbytes += base["table"].numel() * (e + 4)
    ai = flops / nbytes
    if ai < RIDGE:
        roof = {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 3), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / (ms * 1e-3) / 1e12, 3), "peak": PEAK_MFMA_TFLOPS,
                "unit": "TFLOP/s"}
    roof.update({"frac": round(roof["achieved"] / roof["peak"], 4), "traffic": None,
                 "kernel_mean_ms": round(ms, 6), "timing": note})
    rec.update({"ms_per_step": round(ms, 6), "tflops": round(flops / (ms * 1e-3) / 1e12, 4),
                "gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 2), "flops_per_step": flops,
                "algorithmic_bytes_per_step": nbytes, "rotating_input_sets": n_sets, "roofline": roof,
                "pass": "backward (attn_bwd_opt, given the forward's O and log-sum-exp)"})
    del sets, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def copy_floor(torch, nbytes: int, K: int, settle_ms: float):
    """A plain device copy moving ``nbytes`` in all (half read, half written),
    on rotating cold buffers, timed like the attention steps."""
    dev = torch.device("cuda:0")
    n = nbytes // 2 // 2  # f16 elements read (and written) per copy
    n_sets = max(2, math.ceil(512e6 / (4 * n)))
    src = [torch.ones(n, dtype=torch.float16, device=dev) for _ in range(n_sets)]
    dst = [torch.empty_like(src[0]) for _ in range(n_sets)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        dst[i % n_sets].copy_(src[i % n_sets])

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    total_ms, note, g = timed_graph(torch, stream, step, K, settle_ms)
    del g, src, dst
    torch.cuda.empty_cache()
    us = total_ms / K * 1e3
    return {"us": round(us, 3), "bytes_moved": 4 * n, "gb_per_s": round(4 * n / (us * 1e-6) / 1e9, 1),
            "what": f"torch copy_ of {2 * n} bytes of f16 into another buffer (read {2 * n}, write "
                    f"{2 * n}: the headline's algorithmic bytes), {n_sets} rotating buffer pairs, "
                    f"timed like the attention steps"}


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
                    help="GPU time of the untimed launches queued right before the timed ones")
    ap.add_argument("--config", default="C2", help="headline workload")
    ap.add_argument("--extra", default="all",
                    help="comma-separated workloads also timed in this run ('all' or 'none'; "
                         "C2p is C2 with 3 heads of a window per workgroup; C2b, C3b, C4b and "
                         "C5sb are the backward passes of C2, C3, C4 and C5s; C2f8, C5sf8, C5xf8 "
                         "take q, k, v as E4M3 codes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle error checks")
    ap.add_argument("--check-units", type=int, default=16,
                    help="oracle units compared per workload (the headline: all of them)")
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

    need_pool = not (args.no_cpu_baseline and args.no_check) and not args.copy_calibration
    if need_pool:
        # The oracle's worker pool starts before the GPU is initialised.
        from oracle import pool
        pool.start()

    import torch

    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return

    from scaled_dot_product_16_amd import binding
    from scaled_dot_product_16_amd import workloads as W

    binding.lib()
    w = W.WORKLOADS[args.config]
    K = args.steps
    head_units = 0
    if not args.no_check:
        from oracle import pool as opool
        head_units = len(opool.units_of(w))  # the headline is checked on every unit
    rec, inp = run_workload(torch, W, binding, w, K, args.warmup, args.settle_ms, args.no_graph,
                            head_units)
    ms_per_step = rec["ms_per_step"]

    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count, **device_clocks(0),
              "hip": torch.version.hip, "torch": torch.__version__,
              "peaks": {"hbm_GBs": PEAK_HBM_GBS, "bf16_fp16_mfma_TFLOPs": PEAK_MFMA_TFLOPS,
                        "fp32_TFLOPs": PEAK_F32_TFLOPS}}
    line = {
        "metric": METRIC,
        "value": rec["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, N(0,0.02^2) tables)",
        "config": config_of(w),
        "gb_per_s": rec["gb_per_s"],
        "flops_per_step": w.flops,
        "algorithmic_bytes_per_step": w.algorithmic_bytes,
        "rotating_input_sets": rec["rotating_input_sets"],
        "device": device,
        "roofline": rec["roofline"],
    }
    for key in ("max_abs_err", "tol", "err_sample"):
        if key in rec:
            line[key] = rec[key]
    if not args.no_graph:
        line["copy_floor"] = copy_floor(torch, w.algorithmic_bytes, K, args.settle_ms)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
    extra = [] if args.extra == "none" else (ALL + ["C2p"] + BACKWARD + LOW_PRECISION
                                             if args.extra == "all" else args.extra.split(","))
    if extra:
        line["workloads"] = {}
        for key in extra:
            if key == args.config:
                continue
            if key in BACKWARD:  # backward passes
                we = W.WORKLOADS[key[:-1]]
                r = run_backward(torch, W, binding, we, K, args.warmup, args.settle_ms,
                                 0 if args.no_check else 1)
                r["config"] = config_of(we)
                r["dtype"] = we.dtype
                line["workloads"][key] = r
                print(f"# {key} {we.name} backward: {r['ms_per_step'] * 1e3:.2f} us, "
                      f"{r['roofline']['frac']:.3f} of {r['roofline']['bound']} peak"
                      + (f", max abs err {r['max_abs_err']:.2e}" if "max_abs_err" in r else ""),
                      file=sys.stderr, flush=True)
                continue
            # C2p: the Swin-T workload with its 3 heads of a window packed
            # into one workgroup (the packed short-sequence form).
            we = W.WORKLOADS["C2" if key == "C2p" else key]
            fkw = {"window_heads": 3} if key == "C2p" else None
            r, _ = run_workload(torch, W, binding, we, K, args.warmup, args.settle_ms, args.no_graph,
                                0 if args.no_check else args.check_units, fwd_kw=fkw)
            r["config"] = config_of(we)
            if fkw:
                r["config"].update(fkw)
            r["dtype"] = we.dtype
            line["workloads"][key] = r
            print(f"# {key} {we.name}: {r['ms_per_step'] * 1e3:.2f} us, "
                  f"{r['roofline']['frac']:.3f} of {r['roofline']['bound']} peak"
                  + (f", max abs err {r['max_abs_err']:.2e}" if "max_abs_err" in r else ""),
                  file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
