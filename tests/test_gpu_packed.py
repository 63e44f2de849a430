"""GPU parity of the packed short-sequence form: several heads of one window
in one workgroup (attn_fwd_opt, window_heads = 2, 3 or 4), against the fp64
oracle on every output element.

Covers the Swin-T stage-1 workload at full size, Swin-B-like windows with
four heads, every head dim, ragged windows (fewer than 64 queries or keys),
table bias and region mask on and off, the image layout with shift and
zero padding, and a grid of more workgroups than the chip holds.
"""

import sys

import pytest
import torch

from scaled_dot_product_16_amd import workloads as W
from tests.helpers import TOL, check_full, run_gpu, to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scaled_dot_product_16_amd import binding
    binding.lib()


def test_swin_t_stage1_packed():
    w = W.WORKLOADS["C2"]
    say("[packed] C2 at full size, 3 heads per workgroup")
    inp = W.make_inputs(w)
    err = check_full(w, inp, run_gpu(w, to_device(inp), window_heads=3),
                     name="C2 swin_t_stage1_shifted_f16, 3 heads per workgroup")
    say(f"  max abs err {err:.3e} (tol {TOL[w.dtype]:.0e})")


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("hg", [2, 4])
def test_swin_b_like_image_layout(dtype, hg):
    # 4 heads, 56x56 image of 7x7 windows, shift 3, table bias, region mask.
    geom = (56, 56, 7, 7, 3, 3)
    w = W.custom(dtype, B=2 * 64, H=4, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7), mask="shift",
                 layout="image", images=2, window=geom, cfg_id=700 + hg)
    say(f"[packed] {dtype} 4 heads, {hg} per workgroup, image layout {geom}")
    inp = W.make_inputs(w, seed=hg, std_table=0.5)
    check_full(w, inp, run_gpu(w, to_device(inp), window_heads=hg), name=f"packed 4 heads hg={hg} {dtype}")


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("d", [32, 40, 64, 80])
@pytest.mark.parametrize("nq,nk", [(49, 49), (7, 64), (64, 1), (33, 50), (64, 64), (1, 17)])
def test_packed_shapes_no_bias(dtype, d, nq, nk):
    w = W.custom(dtype, B=5, H=6, Nq=nq, Nk=nk, d=d, cfg_id=710 + d)
    say(f"[packed] {dtype} d={d} Nq={nq} Nk={nk}, 3 heads per workgroup")
    inp = W.make_inputs(w, seed=nq * 100 + nk)
    check_full(w, inp, run_gpu(w, to_device(inp), window_heads=3))


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("case", [("table", (7, 7), "none", None), ("table", (5, 9), "none", None),
                                  ("none", None, "shift", (16, 16, 4, 8, 2, 5)),
                                  ("table", (4, 8), "shift", (16, 16, 4, 8, 1, 3))])
def test_packed_bias_and_mask(dtype, case):
    bias, grid, mask, window = case
    if mask == "shift":
        ih, iw, wh, ww = window[:4]
        n, B = wh * ww, 2 * (ih // wh) * (iw // ww)
    else:
        n, B = grid[0] * grid[1], 3
    w = W.custom(dtype, B=B, H=4, Nq=n, Nk=n, d=64, bias=bias, grid=grid, mask=mask, window=window,
                 cfg_id=720)
    say(f"[packed] {dtype} {case}, 2 heads per workgroup")
    inp = W.make_inputs(w, seed=n, std_table=0.5)
    check_full(w, inp, run_gpu(w, to_device(inp), window_heads=2))


@pytest.mark.parametrize("geom", [(15, 13, 7, 7, 3, 3), (20, 25, 4, 8, 2, 5), (14, 14, 7, 7, 0, 0)])
def test_packed_padded_image_layout(geom):
    ih, iw, wh, ww, sh, sw = geom
    ph, pw = -(-ih // wh) * wh, -(-iw // ww) * ww
    nW = (ph // wh) * (pw // ww)
    mask = "shift" if sh or sw else "none"
    w = W.custom(W.F16, B=2 * nW, H=3, Nq=wh * ww, Nk=wh * ww, d=32, bias="table", grid=(wh, ww),
                 mask=mask, layout="image", images=2, window=geom, cfg_id=730)
    say(f"[packed] padded image {geom}, 3 heads per workgroup")
    inp = W.make_inputs(w, seed=sum(geom), std_table=0.5)
    dev = to_device(inp)
    out = run_gpu(w, dev, window_heads=3)
    check_full(w, inp, out)
    # The one-head form gives the same result up to the row-sum rounding
    # (ones column of V on the matrix cores against fp32 sums).
    ref = run_gpu(w, dev, window_heads=1)
    assert (out.float() - ref.float()).abs().max().item() <= TOL[W.F16]


def test_packed_many_workgroups():
    # 24576 windows x 3 heads: 24576 workgroups of 12 waves, more than one
    # pass over the chip.
    w = W.custom(W.F16, B=24576, H=3, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7), cfg_id=740)
    say("[packed] 24576 windows, table bias, 3 heads per workgroup")
    inp = W.make_inputs(w, seed=1, std_table=0.5)
    dev = to_device(inp)
    out = run_gpu(w, dev, window_heads=3)
    ref = run_gpu(w, dev, window_heads=1)
    assert (out.float() - ref.float()).abs().max().item() <= TOL[W.F16]
    # Oracle on the first and last windows of the grid.
    sel = W.custom(W.F16, B=64, H=3, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7), cfg_id=740)
    for lo in (0, w.B - 64):
        part = {k: (v[lo:lo + 64] if k in ("q", "k", "v") else v) for k, v in inp.items()}
        check_full(sel, part, out[lo:lo + 64])
