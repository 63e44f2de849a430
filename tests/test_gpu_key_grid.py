"""GPU parity of the decomposed relative-position bias with the keys on a
grid of their own (SAM's coordinate scalers: the shorter axis stretched onto
the longer one) and with tables stored at another length than the grids
need (resized in the kernel), against the fp64 oracle, every output element.

The half-precision calls take the general relative-position form of the
tiled kernel (the row and contraction forms need equal grids); fp32 calls
take the fp32 kernel.  Ratios are whole (2:1, 1:2), fractional in one or
both directions, and mixed between the two axes.
"""

import sys

import numpy as np
import pytest

from scaled_dot_product_16_amd import workloads as W
from tests.helpers import TOL, check_full, run_gpu, to_device, with_dense_terms

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scaled_dot_product_16_amd import binding
    binding.lib()


CASES = [
    # (dtype, head dim, query grid, key grid, batch, heads)
    (W.BF16, 64, (8, 8), (16, 16), 2, 3),      # keys at twice the resolution
    (W.F16, 64, (14, 14), (7, 7), 2, 2),       # keys at half the resolution
    (W.BF16, 80, (10, 6), (4, 9), 3, 2),       # fractional ratios, opposite per axis
    (W.F16, 32, (9, 14), (14, 9), 2, 2),
    (W.BF16, 40, (20, 20), (12, 30), 1, 2),    # several query and key tiles, ragged
    (W.F16, 64, (1, 7), (3, 5), 4, 2),         # a single query row per image
    (W.BF16, 64, (64, 64), (32, 32), 1, 2),    # SAM's 64x64 grid against a 32x32 one
    (W.BF16, 64, (8, 8), (2, 64), 1, 2),       # a long, thin key grid (Rw of 127 rows)
    (W.F16, 32, (1, 1), (16, 16), 3, 2),       # one query
    (W.F32, 32, (5, 7), (7, 3), 2, 2),
    (W.F32, 64, (6, 6), (12, 4), 1, 2),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_key_grid_relpos(case):
    dtype, d, qg, kg, B, H = CASES[case]
    nq, nk = qg[0] * qg[1], kg[0] * kg[1]
    w = W.custom(dtype, B=B, H=H, Nq=nq, Nk=nk, d=d, bias="relpos", grid=qg, kgrid=kg,
                 cfg_id=560 + case)
    say(f"[key grid relpos] {dtype} d={d} q grid {qg} k grid {kg} B={B} H={H}")
    inp = W.make_inputs(w, seed=case)
    err = check_full(w, inp, run_gpu(w, to_device(inp)))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]:.0e})")


def test_equal_key_grid_matches_no_key_grid():
    # A key grid equal to the query grid is the plain decomposed bias: the
    # library takes the same kernel and must give identical bytes.
    import torch
    from scaled_dot_product_16_amd import binding as Bd

    w = W.custom(W.BF16, B=2, H=2, Nq=196, Nk=196, d=64, bias="relpos", grid=(14, 14),
                 cfg_id=580)
    say("[key grid relpos] explicit equal key grid, 14x14")
    t = to_device(W.make_inputs(w, seed=3))
    a = Bd.fwd(t["q"], t["k"], t["v"], bias=Bd.RelposBias(t["rh"], t["rw"], (14, 14)))
    b = Bd.fwd(t["q"], t["k"], t["v"], bias=Bd.RelposBias(t["rh"], t["rw"], (14, 14), (14, 14)))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_key_grid_tables_too_large_for_lds_are_rejected():
    # Keys on a 2 x 128 grid: the per-query relative terms (130 rows) and the
    # 255-row prologue scratch do not fit one workgroup's LDS next to the K/V
    # tiles, so the launch is refused with E_UNSUPPORTED and nothing runs.
    import torch
    from scaled_dot_product_16_amd import binding as Bd

    w = W.custom(W.BF16, B=1, H=2, Nq=64, Nk=256, d=64, bias="relpos", grid=(8, 8), kgrid=(2, 128),
                 cfg_id=581)
    say("[key grid relpos] 8x8 queries, 2x128 keys: E_UNSUPPORTED, nothing launched")
    dev = to_device(W.make_inputs(w, seed=4))
    assert Bd.check(dev["q"], dev["k"], dev["v"], **W.device_args(w, dev)) == 4
    out = torch.full_like(dev["q"], 7.0)
    with pytest.raises(Bd.AttnError) as e:
        Bd.fwd(dev["q"], dev["k"], dev["v"], out=out, **W.device_args(w, dev))
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_key_grid_relpos_with_additive_mask(dtype):
    # The relative terms on a key grid plus a dense [3, Nq, Nk] mask used as
    # b % 3: both go through the per-score lookup of the general form.
    w = W.custom(dtype, B=6, H=2, Nq=60, Nk=72, d=64 if dtype == W.BF16 else 32, bias="relpos",
                 grid=(6, 10), kgrid=(8, 9), mask="additive", cfg_id=582)
    say(f"[key grid relpos] {dtype} 6x10 queries, 8x9 keys, additive mask [3, 60, 72]")
    inp = with_dense_terms(w, W.make_inputs(w, seed=5), n_mask=3)
    err = check_full(w, inp, run_gpu(w, to_device(inp)))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]:.0e})")


# Tables stored at another length than the grids need (rel_pos_resized):
# resized in the kernel by linear interpolation along the offset axis (end
# rows kept), compared with the oracle, which resizes the table first.
RESIZE_CASES = [
    # (dtype, head dim, query grid, key grid or None, stored Rh rows, stored Rw rows)
    (W.BF16, 64, (14, 14), None, 15, 31),     # SAM windows, tables from other window sizes
    (W.F16, 64, (14, 14), None, 27, 9),
    (W.BF16, 64, (32, 32), None, 127, 127),   # SAM's 64x64 tables on a 32x32 grid
    (W.BF16, 80, (16, 64), None, 63, 255),    # a 64-wide grid: the table form instead of the row form
    (W.F16, 40, (6, 10), (9, 5), 5, 40),      # resize together with a key grid
    (W.BF16, 32, (3, 3), None, 1, 2),         # one- and two-row tables
    (W.F32, 32, (14, 14), None, 15, 31),
    (W.F32, 64, (6, 10), (9, 5), 5, 40),
]


@pytest.mark.parametrize("case", range(len(RESIZE_CASES)))
def test_resized_tables(case):
    import torch

    dtype, d, qg, kg, nh, nw = RESIZE_CASES[case]
    kgr = kg or qg
    nq, nk = qg[0] * qg[1], kgr[0] * kgr[1]
    w = W.custom(dtype, B=2, H=2, Nq=nq, Nk=nk, d=d, bias="relpos", grid=qg, kgrid=kg, cfg_id=590 + case)
    say(f"[resized tables] {dtype} d={d} grid {qg} key grid {kg} stored rows {nh}, {nw}")
    inp = W.make_inputs(w, seed=case)
    std = 1.0 / float(np.sqrt(d))
    inp["rh"] = W.to_dtype(W.normal((nh, d), 590 + case, 3, std), dtype)
    inp["rw"] = W.to_dtype(W.normal((nw, d), 590 + case, 4, std), dtype)
    err = check_full(w, inp, run_gpu(w, to_device(inp)), name=f"resized tables {qg}/{kg} rows {nh},{nw} d={d}")
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert torch.cuda.is_available()


def test_resized_tables_image_layout():
    # SAM windows read from the unpadded image with resized tables.
    geom = (30, 20, 14, 14, 0, 0)
    w = W.custom(W.BF16, B=2 * 6, H=2, Nq=196, Nk=196, d=64, bias="relpos", grid=(14, 14),
                 layout="image", images=2, window=geom, cfg_id=599)
    say(f"[resized tables] image layout {geom}, stored rows 21, 33")
    inp = W.make_inputs(w, seed=9)
    inp["rh"] = W.to_dtype(W.normal((21, 64), 599, 3, 0.125), W.BF16)
    inp["rw"] = W.to_dtype(W.normal((33, 64), 599, 4, 0.125), W.BF16)
    err = check_full(w, inp, run_gpu(w, to_device(inp)), name="resized tables, image layout")
    say(f"  max abs err {err:.3e} (tol {TOL[W.BF16]:.0e})")
