"""GPU: the per-row log-sum-exp output of the forward (attn_options_t.lse)
against the oracle's, for every forward form, and the backward that takes
the forward's O and log-sum-exp (attn_bwd_opt) against the oracle and the
plain backward.

Tolerance: the forward's max-abs bound for the compute dtype (the log-sum-exp
is of the same logits, whose relative-position terms some forms carry in the
element type).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_16_amd import binding as Bd
from scaled_dot_product_16_amd import workloads as W
from tests.helpers import TOL, check_full, oracle_arrays, record, to_device, with_dense_terms

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Bd.lib()


def run_with_lse(w, dev):
    lse = torch.full(tuple(w.q_shape[:3]), float("nan"), dtype=torch.float32, device="cuda")
    out = Bd.fwd(dev["q"], dev["k"], dev["v"], lse=lse, **W.device_args(w, dev))
    torch.cuda.synchronize()
    return out, lse


def check_lse(w, inp, lse, name=None):
    ref = oracle.run_workload_logsumexp(w, oracle_arrays(inp))
    got = lse.detach().double().cpu().numpy()
    if w.layout == "image":
        # Every real pixel has an entry (padding tokens have none).
        assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref)))
    tol = TOL[w.dtype]
    if name:
        record(name, w.dtype, err, tol, got.size)
    assert err <= tol, f"lse: max abs err {err:.3e} > {tol:.1e}"
    return err


CASES = [
    # (label, workload kwargs, table std)
    ("window, table + shift, image layout", dict(dtype=W.F16, B=2 * 64, H=3, Nq=49, Nk=49, d=32, bias="table",
                                                grid=(7, 7), mask="shift", layout="image", images=2,
                                                window=(56, 56, 7, 7, 3, 3)), 0.5),
    ("window, ragged", dict(dtype=W.BF16, B=5, H=2, Nq=33, Nk=50, d=64), 0.02),
    ("table form, additive bias and mask", dict(dtype=W.F16, B=3, H=2, Nq=300, Nk=300, d=64, bias="additive",
                                               mask="additive"), 0.02),
    ("two-tile form (cross-attention)", dict(dtype=W.F16, B=2, H=4, Nq=1000, Nk=77, d=40), 0.02),
    ("two-tile form, three query tiles per workgroup", dict(dtype=W.F16, B=40, H=8, Nq=1000, Nk=77, d=40), 0.02),
    # The contraction form carries the relative-position terms through the
    # matrix cores in the element type (error ~ |bias| * 2^-9 in bf16): its
    # tables are drawn at the workloads' N(0, 0.02^2).
    ("contraction form (14x14 relpos)", dict(dtype=W.BF16, B=4, H=3, Nq=196, Nk=196, d=64, bias="relpos",
                                            grid=(14, 14)), 0.02),
    ("row form (4x64 relpos)", dict(dtype=W.BF16, B=2, H=2, Nq=256, Nk=256, d=80, bias="relpos",
                                   grid=(4, 64)), 0.5),
    ("two-group form (64x64 relpos)", dict(dtype=W.BF16, B=1, H=2, Nq=4096, Nk=4096, d=64, bias="relpos",
                                          grid=(64, 64)), 0.125),
    ("table form, key grid", dict(dtype=W.BF16, B=2, H=2, Nq=100, Nk=64, d=64, bias="relpos", grid=(10, 10),
                                  kgrid=(8, 8)), 0.5),
    ("tiled, padded image (SAM windows)", dict(dtype=W.BF16, B=25, H=2, Nq=196, Nk=196, d=64, bias="relpos",
                                             grid=(14, 14), layout="image", images=1,
                                             window=(64, 64, 14, 14, 0, 0)), 0.02),
    ("8-bit inputs, window", dict(dtype=W.F16, B=2 * 64, H=3, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7),
                                  mask="shift", layout="image", images=2, window=(56, 56, 7, 7, 3, 3),
                                  qkv="e4m3"), 0.5),
    ("8-bit inputs, tiled", dict(dtype=W.F16, B=2, H=2, Nq=500, Nk=500, d=40, qkv="e4m3"), 0.02),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forward_lse(case):
    label, kw, std = CASES[case]
    w = W.custom(cfg_id=300 + case, **kw)
    say(f"[lse] {label}")
    inp = with_dense_terms(w, W.make_inputs(w, seed=case, std_table=std), n_bias=2, n_mask=3)
    dev = to_device(inp)
    out, lse = run_with_lse(w, dev)
    check_full(w, inp, out)
    # The output does not change when the log-sum-exp is also written.
    ref_out = Bd.fwd(dev["q"], dev["k"], dev["v"], **W.device_args(w, dev))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    err = check_lse(w, inp, lse, name=f"lse {label}")
    say(f"  max abs err {err:.3e}")


# (label, workload kwargs, table std).  The 14x14 grid's forward runs the
# contraction form, whose O and log-sum-exp carry the bias in the element
# type: its tables use the workloads' N(0, 0.02^2).
BWD_CASES = [
    ("SD-style self-attention", dict(dtype=W.F16, B=2, H=2, Nq=1000, Nk=1000, d=40), 0.5),
    ("cross-attention", dict(dtype=W.BF16, B=2, H=2, Nq=300, Nk=77, d=64), 0.5),
    ("14x14 relpos", dict(dtype=W.BF16, B=4, H=3, Nq=196, Nk=196, d=64, bias="relpos", grid=(14, 14)), 0.02),
    ("4x64 relpos", dict(dtype=W.BF16, B=2, H=2, Nq=256, Nk=256, d=64, bias="relpos", grid=(4, 64)), 0.5),
    ("window (statistics ignored)", dict(dtype=W.F16, B=6, H=3, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7)),
     0.5),
]


@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_backward_with_forward_statistics(case):
    label, kw, std = BWD_CASES[case]
    w = W.custom(cfg_id=320 + case, **kw)
    say(f"[bwd+lse] {label}")
    inp = W.make_inputs(w, seed=case, std_table=std)
    inp["dout"] = W.to_dtype(W.normal(w.q_shape, w.cfg_id, 7, 1.0, case), w.dtype)
    dev = to_device(inp)
    out, lse = run_with_lse(w, dev)
    kwd = W.device_args(w, dev)
    g_plain = Bd.bwd(dev["q"], dev["k"], dev["v"], dev["dout"], **kwd)
    g_stat = Bd.bwd(dev["q"], dev["k"], dev["v"], dev["dout"], out=out, lse=lse, **kwd)
    torch.cuda.synchronize()
    ref = oracle.run_workload_backward(w, oracle_arrays(inp))
    names = ["dq", "dk", "dv"]
    got = list(g_stat[:3])
    if w.bias == "relpos":
        names += ["drh", "drw"]
        got += list(g_stat[3])
    elif w.bias == "table":
        names += ["dtable"]
        got += [g_stat[3]]
    for key, g in zip(names, got):
        r = ref[key]
        gg = g.detach().double().cpu().numpy()
        err = float(np.max(np.abs(gg - r)))
        tol = TOL[w.dtype] * max(1.0, float(np.max(np.abs(r))))
        record(f"bwd with statistics, {label} {key}", w.dtype, err, tol, gg.size)
        assert err <= tol, f"{key}: max abs err {err:.3e} > {tol:.3e}"
    if w.Nq <= 64 and w.Nk <= 64:
        # The window path recomputes P and ignores the statistics.
        for x, y in zip(g_plain[:3], g_stat[:3]):
            assert torch.equal(x, y)
