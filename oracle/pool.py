"""Process-pool evaluation of the fp64 oracle over (batch item, head) units.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and by the ``cpu_baseline`` leg
of ``bench.py``; never by the product path.  This module holds no attention
arithmetic: every unit is computed by :func:`oracle.attention.attention` on
that unit's own slice of the inputs, exactly as the serial oracle would
compute it (softmax rows are independent, and so are (batch item, head)
units).  It only splits the work, moves arrays and collects results.

Workers are forked from a fork server that is started before the calling
process touches the GPU (call :func:`start` early), so no worker inherits a
GPU context or device file.  Each worker runs single-threaded BLAS, so the
pool's parallelism is its process count, which is reported.

Inputs travel through ``.npy`` files in a temporary directory (float32 holds
every f16/bf16 value and every 8-bit code exactly; f32 inputs are stored as
they are), opened by the workers as read-only memory maps.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile
import time
from typing import Dict, Optional, Sequence

import numpy as np

_CTX = None
MAX_WORKERS = 16


def workers_available() -> int:
    """Processes the pool uses: the host cores this process may run on, at
    most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


def start() -> None:
    """Start the fork server (a fresh interpreter that preloads numpy and the
    oracle, with single-threaded BLAS).  Must run before this process
    initialises the GPU: the server is a child process started then, and
    every worker is forked from it, never from a process holding a GPU
    context.  Raises if the GPU is already initialised."""
    global _CTX
    if _CTX is not None:
        return
    import sys
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_initialized():
        raise RuntimeError("oracle.pool.start() must run before the GPU is initialised")
    ctx = mp.get_context("forkserver")
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        ctx.set_forkserver_preload(["numpy", "oracle.attention", "oracle.pool"])
        from multiprocessing import forkserver
        forkserver.ensure_running()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    _CTX = ctx


# ---------------------------------------------------------------------------
# Worker side
# ---------------------------------------------------------------------------

_W: dict = {}


def _init(paths: Dict[str, str], spec: dict) -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    _W.clear()
    _W["arrays"] = {k: np.load(p, mmap_mode="r") for k, p in paths.items()}
    _W["spec"] = spec


def _unit_inputs(b: int, h: int, drop: Optional[str] = None):
    """The oracle's arguments for unit (b, h): that unit's q, k, v and the
    bias and mask terms it uses (table column h, dense slice b mod n).  In
    the image layout a unit is (image b, head h): its windows, shift and
    region mask lie inside the image, so the image alone is evaluated."""
    from oracle.attention import Bias, Mask

    A, S = _W["arrays"], _W["spec"]
    f = lambda x: np.asarray(x, dtype=np.float64)
    q = f(A["q"][b:b + 1, h:h + 1])
    k = f(A["k"][b:b + 1, h:h + 1])
    v = f(A["v"][b:b + 1, h:h + 1])
    if S.get("qkv", "same") == "e4m3":
        # 8-bit inputs: the arrays hold E4M3 codes, "descale" their scales.
        from oracle.attention import dequantize_e4m3
        s = np.asarray(A["descale"], dtype=np.float64).reshape(-1)
        q, k, v = (dequantize_e4m3(x, s[i]) for i, x in enumerate((q, k, v)))
    bias = Bias("none")
    if S["bias"] == "table":
        bias = Bias("table", grid=S["grid"], table=f(A["table"][:, h:h + 1]))
    elif S["bias"] == "relpos":
        rh, rw = f(A["rh"]), f(A["rw"])
        # drop="rh" / "rw": that table's term left out (zero table), for
        # tests that show a check can see a missing term.
        if drop == "rh":
            rh = np.zeros_like(rh)
        elif drop == "rw":
            rw = np.zeros_like(rw)
        bias = Bias("relpos", grid=S["grid"], kgrid=S.get("kgrid"), rh=rh, rw=rw)
    elif S["bias"] == "additive":
        a = A["bias_add"]
        bias = Bias("additive", add=f(a[b % a.shape[0]][None]))
    if drop == "bias":
        bias = Bias("none")
    mask = Mask("none")
    if S["mask"] == "additive":
        a = A["mask_add"]
        mask = Mask("additive", add=f(a[b % a.shape[0]][None]))
    elif S["mask"] == "shift":
        if S.get("layout") != "image":
            raise ValueError("the pooled oracle takes the region mask in the image layout only")
        mask = Mask("shift", window=tuple(S["window"]))
    return q, k, v, bias, mask


def _evaluate(q, k, v, bias, mask):
    from oracle.attention import attention, attention_image

    S = _W["spec"]
    if S.get("layout") == "image":
        return attention_image(q, k, v, tuple(S["window"]), bias, mask)
    return attention(q, k, v, bias, mask)


def _unit_job(job):
    """One unit: the oracle's output rows compared with the GPU output."""
    b, h, drops = job
    t0 = time.perf_counter()
    q, k, v, bias, mask = _unit_inputs(b, h)
    ref = _evaluate(q, k, v, bias, mask)[0, 0]
    res = {"b": b, "h": h, "ref_absmax": float(np.max(np.abs(ref)))}
    got = _W["arrays"].get("out")
    if got is not None:
        g = np.asarray(got[b, h], dtype=np.float64)
        res["err"] = float(np.max(np.abs(g - ref))) if np.all(np.isfinite(g)) else float("inf")
    # Distance of the full result from the result without a term (the size
    # of the change a check must be able to see).
    for d in drops:
        qd, kd, vd, bd, md = _unit_inputs(b, h, drop=d)
        res["delta_" + d] = float(np.max(np.abs(_evaluate(qd, kd, vd, bd, md)[0, 0] - ref)))
    res["seconds"] = time.perf_counter() - t0
    return res


def _timing_job(job):
    """One unit of the oracle, timed (no comparison)."""
    b, h = job
    q, k, v, bias, mask = _unit_inputs(b, h)
    t0 = time.perf_counter()
    _evaluate(q, k, v, bias, mask)
    return time.perf_counter() - t0


# ---------------------------------------------------------------------------
# Caller side
# ---------------------------------------------------------------------------

def spec_of(w) -> dict:
    """The description a pool needs of a workload record."""
    return {"bias": w.bias, "grid": w.grid, "kgrid": getattr(w, "kgrid", None), "mask": w.mask,
            "layout": w.layout, "window": w.window, "qkv": getattr(w, "qkv", "same")}


def units_of(w) -> list:
    """All units of a workload: (batch item, head), or (image, head) in the
    image layout."""
    nb = w.images if w.layout == "image" else w.B
    return [(b, h) for b in range(nb) for h in range(w.H)]


class UnitPool:
    """Arrays of one workload written once; units mapped over a worker pool.

    ``arrays``: q, k, v [B, H, N, d] and the workload's tables / dense terms
    (numpy or torch CPU tensors); ``out`` optionally the GPU output to compare
    with.  ``spec``: dict with bias, grid, kgrid, mask, layout, window (the
    workload's description; see :func:`spec_of`).
    """

    def __init__(self, arrays: dict, spec: dict, workers: Optional[int] = None):
        start()
        self.dir = tempfile.mkdtemp(prefix="oracle_pool_")
        self.paths = {}
        for name, x in arrays.items():
            if x is None:
                continue
            if hasattr(x, "detach"):
                import torch
                x = x.detach().to("cpu")
                x = x.to(torch.float32) if x.dtype != torch.float64 else x
                x = x.numpy()
            x = np.ascontiguousarray(x)
            if x.dtype not in (np.float32, np.float64):
                x = x.astype(np.float32)
            p = os.path.join(self.dir, name + ".npy")
            np.save(p, x)
            self.paths[name] = p
        self.spec = dict(spec)
        self.workers = workers or workers_available()
        # A worker that dies makes the executor raise (BrokenProcessPool)
        # instead of being replaced, so a failure cannot turn into a hang.
        from concurrent.futures import ProcessPoolExecutor
        self.pool = ProcessPoolExecutor(self.workers, mp_context=_CTX, initializer=_init,
                                        initargs=(self.paths, self.spec))

    def compare(self, units: Sequence, drops: Dict[tuple, Sequence[str]] = None) -> list:
        """Per-unit results for [(b, h), ...]: max-abs error against ``out``
        and, for units listed in ``drops``, the change from leaving a term
        out."""
        drops = drops or {}
        jobs = [(b, h, tuple(drops.get((b, h), ()))) for (b, h) in units]
        return list(self.pool.map(_unit_job, jobs))

    def time_units(self, units: Sequence) -> float:
        """Wall seconds to evaluate the oracle on ``units`` across the pool
        (input slicing excluded only inside each unit's own timer; the wall
        clock covers the whole map)."""
        t0 = time.perf_counter()
        list(self.pool.map(_timing_job, list(units)))
        return time.perf_counter() - t0

    def close(self):
        if self.pool is not None:
            self.pool.shutdown(wait=True)
            self.pool = None
        shutil.rmtree(self.dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
