"""Shared helpers of the parity tests: run a workload on the GPU through the
C ABI and evaluate the oracle on the very same (dtype-rounded) inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from scaled_dot_product_16_amd import workloads as W

# Max-abs error bounds on N(0,1) inputs, per dtype.
TOL = {W.F32: 1e-5, W.F16: 5e-3, W.BF16: 2e-2}


def with_dense_terms(w: W.Workload, inp: dict, seed: int = 0, n_bias: int = 1, n_mask: int = 1,
                     scale: float = 1.0) -> dict:
    """Add dense additive bias/mask tensors (drawn like the rest) when ``w`` needs them."""
    if w.bias == "additive":
        inp["bias_add"] = W.to_dtype(W.normal((n_bias, w.Nq, w.Nk), w.cfg_id, 5, scale, seed), w.dtype)
    if w.mask == "additive":
        inp["mask_add"] = W.to_dtype(W.normal((n_mask, w.Nq, w.Nk), w.cfg_id, 6, scale, seed), w.dtype)
    return inp


def to_device(inp: dict, device="cuda") -> dict:
    return {k: v.to(device) for k, v in inp.items()}


def run_gpu(w: W.Workload, dev: dict, out=None, **override) -> torch.Tensor:
    from scaled_dot_product_16_amd import binding

    kw = W.device_args(w, dev)
    kw.update(override)
    o = binding.fwd(dev["q"], dev["k"], dev["v"], out=out, **kw)
    torch.cuda.synchronize()
    return o


def oracle_arrays(inp: dict) -> dict:
    return {k: v.to(torch.float64).numpy() for k, v in inp.items()}


def sample_select(w: W.Workload, n_pairs: int = 6, n_rows: int = 40, seed: int = 0):
    """(b, h, rows) samples spanning first/last items, tile boundaries and random rows."""
    rng = np.random.default_rng(1000 + seed)
    pairs = {(0, 0), (w.B - 1, w.H - 1)}
    while len(pairs) < min(n_pairs, w.B * w.H):
        pairs.add((int(rng.integers(w.B)), int(rng.integers(w.H))))
    fixed = [r for r in (0, 1, 63, 64, 127, 128, 255, 256, w.Nq - 2, w.Nq - 1) if 0 <= r < w.Nq]
    sel = []
    for (b, h) in sorted(pairs):
        rows = np.unique(np.concatenate([fixed, rng.integers(0, w.Nq, n_rows)]))
        sel.append((b, h, rows))
    return sel


def max_abs_err(got: np.ndarray, ref: np.ndarray) -> float:
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def record(name: str, dtype: str, err: float, tol: float, elements: int, **extra):
    """Keep a compared case's max-abs error for the end-of-run summary."""
    from tests.parity_log import RECORDS

    RECORDS.append({"name": name, "dtype": dtype, "err": float(err), "tol": float(tol),
                           "elements": int(elements), **extra})


def check_full(w: W.Workload, inp: dict, out: torch.Tensor, tol=None, name=None):
    ref = oracle.run_workload(w, oracle_arrays(inp))
    got = out.detach().to("cpu", torch.float64).numpy()
    err = max_abs_err(got, ref)
    tol = TOL[w.dtype] if tol is None else tol
    if name:
        record(name, w.dtype, err, tol, got.size)
    assert err <= tol, f"{w.key}: max abs err {err:.3e} > {tol:.1e}"
    return err


def check_full_pooled(w: W.Workload, inp: dict, out: torch.Tensor, name: str, tol=None,
                      drops=None):
    """Every output element against the oracle, the (batch item, head) units
    (image layout: (image, head)) spread over a process pool.

    ``drops``: {(b, h): ("rh", "rw", "bias")}: for those units the oracle is
    also evaluated with that term left out, and the returned dict holds the
    smallest such change (``delta_<term>``), so a test can assert that the
    check would see a missing term.
    """
    from oracle import pool

    tol = TOL[w.dtype] if tol is None else tol
    arrays = dict(inp, out=out.detach().to("cpu"))
    units = pool.units_of(w)
    with pool.UnitPool(arrays, pool.spec_of(w)) as P:
        res = P.compare(units, drops=drops)
    err = max(r["err"] for r in res)
    summary = {"err": err, "units": len(res)}
    for key in ("delta_rh", "delta_rw", "delta_bias"):
        vals = [r[key] for r in res if key in r]
        if vals:
            summary[key] = min(vals)
    record(name, w.dtype, err, tol, out.numel(),
           **{k: v for k, v in summary.items() if k.startswith("delta")})
    worst = max(res, key=lambda r: r["err"])
    assert err <= tol, f"{name}: max abs err {err:.3e} > {tol:.1e} (b={worst['b']}, h={worst['h']})"
    return summary


def check_sampled(w: W.Workload, inp: dict, out: torch.Tensor, select, tol=None):
    arrs = oracle_arrays(inp)
    refs = oracle.run_workload(w, arrs, select=select)
    tol = TOL[w.dtype] if tol is None else tol
    worst = 0.0
    for (b, h, rows), ref in zip(select, refs):
        got = out[b, h, torch.as_tensor(rows, device=out.device)].to("cpu", torch.float64).numpy()
        err = max_abs_err(got, ref)
        worst = max(worst, err)
        assert err <= tol, f"{w.key} b={b} h={h}: max abs err {err:.3e} > {tol:.1e}"
    return worst
