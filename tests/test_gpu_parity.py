"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every workload is compared element by element at full size (SAM global and
SD with the oracle's (batch item, head) units spread over a process pool).
The decomposed relative position on the 64x64 grid is also run at full size
with tables large enough that leaving out either term moves the output by
more than ten times the measured error.  Reduced sizes sweep head dims,
dtypes, ragged tiles, every bias and mask kind and both layouts.  Max-abs
tolerances: f32 1e-5, f16 5e-3, bf16 2e-2.
"""

import sys

import numpy as np
import pytest
import torch

from scaled_dot_product_16_amd import workloads as W
from tests.helpers import (TOL, check_full, check_full_pooled, run_gpu, to_device,
                           with_dense_terms)

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scaled_dot_product_16_amd import binding
    binding.lib()  # fails loudly if the library is missing


# ---------------------------------------------------------------------------
# The workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("key", ["C1", "C2", "C3", "C3i"])
def test_workload_full(key):
    w = W.WORKLOADS[key]
    say(f"[parity full] {key} {w.name}")
    inp = W.make_inputs(w)
    out = run_gpu(w, to_device(inp))
    err = check_full(w, inp, out, name=f"{key} {w.name}")
    say(f"  max abs err {err:.3e} (tol {TOL[w.dtype]:.0e})")


@pytest.mark.parametrize("key", ["C4", "C4h", "C5s", "C5x"])
def test_workload_full_pooled(key):
    # Every output element; the oracle's units run in a process pool.
    w = W.WORKLOADS[key]
    say(f"[parity full, pooled oracle] {key} {w.name}")
    inp = W.make_inputs(w)
    out = run_gpu(w, to_device(inp))
    res = check_full_pooled(w, inp, out, name=f"{key} {w.name}")
    say(f"  max abs err {res['err']:.3e} over {res['units']} units (tol {TOL[w.dtype]:.0e})")


@pytest.mark.parametrize("key", ["C4", "C4h"])
def test_global_relpos_bias_is_seen(key):
    # SAM global shapes at full size (the two-group kernel through every
    # grid row) with Rh and Rw drawn at N(0, 1/d), so q.Rh and q.Rw are
    # N(0, 1) per term.  On a few units the oracle is also evaluated with Rh
    # and with Rw left out: the measured error must be at most a tenth of
    # either change, so a kernel that lost a term would fail.
    w = W.WORKLOADS[key]
    std = 1.0 / float(np.sqrt(w.d))
    say(f"[parity full, relpos tables N(0, 1/d)] {key} shape")
    inp = W.make_inputs(w, seed=11, std_table=std)
    out = run_gpu(w, to_device(inp))
    drops = {u: ("rh", "rw") for u in [(0, 0), (w.B // 2, w.H // 3), (w.B - 1, w.H - 1), (3, 5)]}
    res = check_full_pooled(w, inp, out, name=f"{key} shape, relpos tables std 1/sqrt(d)",
                            drops=drops)
    say(f"  max abs err {res['err']:.3e}; without Rh {res['delta_rh']:.3e}, "
        f"without Rw {res['delta_rw']:.3e}")
    assert res["err"] <= 0.1 * min(res["delta_rh"], res["delta_rw"])


# ---------------------------------------------------------------------------
# Reduced-size sweeps (several tiles and ragged tails)
# ---------------------------------------------------------------------------

# (300, 1100): long key range with a ragged last key tile and a partial
# query tile.
SHAPES = [(1, 1), (7, 300), (300, 77), (129, 64), (200, 200), (64, 1), (300, 1100)]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
@pytest.mark.parametrize("d", [32, 40, 64, 80])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_plain_shapes(dtype, d, nq, nk):
    w = W.custom(dtype, B=2, H=3, Nq=nq, Nk=nk, d=d, cfg_id=100 + d)
    say(f"[sweep] {dtype} d={d} Nq={nq} Nk={nk}")
    inp = W.make_inputs(w, seed=nq * 1000 + nk)
    check_full(w, inp, run_gpu(w, to_device(inp)))


BIAS_CASES = [
    # (bias, grid, mask, window)
    ("table", (7, 7), "none", None),
    ("table", (5, 9), "none", None),
    ("relpos", (6, 10), "none", None),
    ("relpos", (14, 14), "none", None),
    ("relpos", (3, 50), "none", None),
    ("relpos", (17, 64), "none", None),  # 64-wide grid, long key range (two-group schedule)
    ("relpos", (16, 64), "none", None),  # 64-wide grid at the two-group schedule's 1024-key threshold
    ("relpos", (2, 64), "none", None),  # 64-wide grid, exactly two key tiles
    ("additive", None, "none", None),
    ("none", None, "additive", None),
    ("additive", None, "additive", None),
    ("table", (7, 7), "shift", (28, 21, 7, 7, 3, 2)),
    # a table lookup together with a dense term on the window path
    ("table", (7, 7), "additive", None),
    ("additive", None, "shift", (14, 14, 7, 7, 3, 3)),
    ("table", (8, 8), "additive", None),
    ("none", None, "shift", (16, 16, 4, 8, 2, 5)),
    ("relpos", (4, 8), "shift", (16, 16, 4, 8, 1, 3)),
]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
@pytest.mark.parametrize("case", range(len(BIAS_CASES)))
def test_bias_and_mask_kinds(dtype, case):
    bias, grid, mask, window = BIAS_CASES[case]
    if mask == "shift":
        ih, iw, wh, ww = window[:4]
        n = wh * ww
        B = 2 * (ih // wh) * (iw // ww)
    else:
        n = grid[0] * grid[1] if grid else 150
        B = 3
    d = 64 if dtype != W.F32 else 32
    w = W.custom(dtype, B=B, H=2, Nq=n, Nk=n, d=d, bias=bias, grid=grid, mask=mask,
                 window=window, cfg_id=200 + case)
    say(f"[bias/mask] {dtype} {bias} {grid} {mask} {window} B={B} N={n}")
    inp = with_dense_terms(w, W.make_inputs(w, seed=case), n_bias=2, n_mask=3)
    check_full(w, inp, run_gpu(w, to_device(inp)))


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("d", [32, 40, 80])
@pytest.mark.parametrize("grid", [(17, 64), (16, 64), (2, 64)])
def test_relpos_64_wide_grids_head_dims(dtype, d, grid):
    # The 64-wide row form at the head dims the other sweeps leave to the
    # general forms: above and at the two-group schedule's key threshold and
    # at exactly two key tiles.  Tables at N(0, 1/d) make the bias large.
    n = grid[0] * grid[1]
    w = W.custom(dtype, B=2, H=2, Nq=n, Nk=n, d=d, bias="relpos", grid=grid, cfg_id=250 + d)
    say(f"[relpos 64-wide] {dtype} d={d} grid {grid}")
    inp = W.make_inputs(w, seed=grid[0], std_table=1.0 / float(np.sqrt(d)))
    check_full(w, inp, run_gpu(w, to_device(inp)), name=f"relpos grid {grid} d={d}")


@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
@pytest.mark.parametrize("n", [65, 100, 128])
def test_two_key_tiles_dense_terms(dtype, n):
    # Keys spanning two tiles (both loaded up front), with dense additive bias
    # and mask, one of each per batch item group.
    d = 64 if dtype != W.F32 else 32
    w = W.custom(dtype, B=6, H=2, Nq=n, Nk=n, d=d, bias="additive", mask="additive", cfg_id=600 + n)
    say(f"[two tiles] {dtype} N={n}")
    inp = with_dense_terms(w, W.make_inputs(w, seed=n), n_bias=2, n_mask=3)
    check_full(w, inp, run_gpu(w, to_device(inp)))


@pytest.mark.parametrize("dtype,d", [(W.F16, 32), (W.F16, 40), (W.BF16, 64), (W.BF16, 80)])
def test_two_tiles_several_query_tiles_per_workgroup(dtype, d):
    # Cross-attention to 77 keys (the two-tile form, batched layout) with
    # enough (batch item, head) units that each workgroup walks 3 or 4
    # consecutive query tiles (K and V kept in LDS, the next tile's Q loaded
    # during the current one; at d = 64 one tile per workgroup); 1000
    # queries leave a ragged last tile, and at d = 32, 40 the last workgroup
    # of a unit holds fewer tiles than the first.
    w = W.custom(dtype, B=40, H=8, Nq=1000, Nk=77, d=d, cfg_id=700 + d)
    say(f"[two tiles, several query tiles per workgroup] {dtype} d={d}")
    inp = W.make_inputs(w, seed=d)
    res = check_full_pooled(w, inp, run_gpu(w, to_device(inp)), name=f"two tiles, 3-4 query tiles per workgroup d={d}")
    say(f"  max abs err {res['err']:.3e} over {res['units']} units")


@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
@pytest.mark.parametrize("geom", [(14, 14, 7, 7, 3, 3), (16, 32, 4, 8, 2, 5), (12, 12, 6, 6, 0, 0)])
def test_image_layout(dtype, geom):
    ih, iw, wh, ww, sh, sw = geom
    nW = (ih // wh) * (iw // ww)
    mask = "shift" if sh or sw else "none"
    d = 32
    w = W.custom(dtype, B=2 * nW, H=3, Nq=wh * ww, Nk=wh * ww, d=d, bias="table", grid=(wh, ww),
                 mask=mask, layout="image", images=2, window=geom, cfg_id=300)
    say(f"[image] {dtype} {geom}")
    inp = W.make_inputs(w, seed=sum(geom))
    dev = to_device(inp)
    out = run_gpu(w, dev)
    check_full(w, inp, out)

    # Same result, bit for bit, from explicitly shifted and partitioned inputs
    # in the batched layout.
    def part(x):
        x = x.reshape(2, 3, ih, iw, d)
        x = torch.roll(x, shifts=(-sh, -sw), dims=(2, 3))
        x = x.reshape(2, 3, ih // wh, wh, iw // ww, ww, d).permute(0, 2, 4, 1, 3, 5, 6)
        return x.reshape(2 * nW, 3, wh * ww, d).contiguous()

    wb = W.custom(dtype, B=2 * nW, H=3, Nq=wh * ww, Nk=wh * ww, d=d, bias="table", grid=(wh, ww),
                  mask=mask, layout="batched", window=geom, cfg_id=300)
    devb = dict(dev, q=part(dev["q"]), k=part(dev["k"]), v=part(dev["v"]))
    outb = run_gpu(wb, devb)
    assert torch.equal(part(out), outb)


# Images that are not a whole number of windows: zero padding at the bottom
# and right is folded into the addressing.  (geometry, bias, head dim):
# 49-token windows (window kernel) with the region mask, 32-token windows,
# 81-token windows with table bias and shift (tiled kernel, table path) and
# SAM-style 14x14 windows with the decomposed relative position.
PADDED = [((15, 13, 7, 7, 3, 3), "table", 32), ((20, 25, 4, 8, 2, 5), "table", 32),
          ((20, 20, 9, 9, 4, 4), "table", 64), ((30, 20, 14, 14, 0, 0), "relpos", 64)]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
@pytest.mark.parametrize("case", range(len(PADDED)))
def test_padded_image_layout(dtype, case):
    geom, bias, d = PADDED[case]
    ih, iw, wh, ww, sh, sw = geom
    ph, pw = -(-ih // wh) * wh, -(-iw // ww) * ww
    nW = (ph // wh) * (pw // ww)
    mask = "shift" if sh or sw else "none"
    w = W.custom(dtype, B=2 * nW, H=3, Nq=wh * ww, Nk=wh * ww, d=d, bias=bias, grid=(wh, ww),
                 mask=mask, layout="image", images=2, window=geom, cfg_id=310 + case)
    say(f"[padded image] {dtype} {geom} {bias} d={d}")
    inp = W.make_inputs(w, seed=sum(geom))
    dev = to_device(inp)
    out = run_gpu(w, dev)
    check_full(w, inp, out)

    # Bit for bit the same as explicitly padded, shifted and partitioned
    # inputs in the batched layout (padding rows are zeros there).
    def part(x):
        x = x.reshape(2, 3, ih, iw, d)
        x = torch.nn.functional.pad(x, (0, 0, 0, pw - iw, 0, ph - ih))
        x = torch.roll(x, shifts=(-sh, -sw), dims=(2, 3))
        x = x.reshape(2, 3, ph // wh, wh, pw // ww, ww, d).permute(0, 2, 4, 1, 3, 5, 6)
        return x.reshape(2 * nW, 3, wh * ww, d).contiguous()

    wb = W.custom(dtype, B=2 * nW, H=3, Nq=wh * ww, Nk=wh * ww, d=d, bias=bias, grid=(wh, ww),
                  mask=mask, layout="batched", window=geom, cfg_id=310 + case)
    devb = dict(dev, q=part(dev["q"]), k=part(dev["k"]), v=part(dev["v"]))
    outb = run_gpu(wb, devb)
    real = part(torch.ones(2, 3, ih * iw, d, device=out.device)).bool()
    assert torch.equal(part(out)[real], outb[real])


@pytest.mark.parametrize("geom", [(64, 64, 64, 64, 0, 0), (60, 62, 64, 64, 0, 0)])
def test_image_layout_global_relpos(geom):
    # One 64x64 window per image: SAM global attention in the image layout
    # (the 64-wide relative-position row form), also on a padded grid.
    w = W.custom(W.BF16, B=1, H=2, Nq=4096, Nk=4096, d=64, bias="relpos", grid=(64, 64),
                 layout="image", images=1, window=geom, cfg_id=320)
    say(f"[image global relpos] {geom}")
    inp = W.make_inputs(w, seed=3)
    err = check_full(w, inp, run_gpu(w, to_device(inp)))
    say(f"  max abs err {err:.3e} (tol {TOL[W.BF16]:.0e})")


# ---------------------------------------------------------------------------
# Invariants and special cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
def test_single_key_returns_v0(dtype):
    w = W.custom(dtype, B=2, H=2, Nq=100, Nk=1, d=64 if dtype != W.F32 else 32, cfg_id=400)
    inp = W.make_inputs(w)
    out = run_gpu(w, to_device(inp))
    assert torch.equal(out.cpu(), inp["v"].expand_as(out))


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_constant_v_gives_constant_output(dtype):
    w = W.custom(dtype, B=1, H=2, Nq=130, Nk=333, d=40, cfg_id=401)
    inp = W.make_inputs(w)
    inp["v"] = torch.ones_like(inp["v"])
    out = run_gpu(w, to_device(inp)).float()
    assert (out - 1).abs().max().item() <= TOL[dtype]


def test_deterministic_and_strided_inputs():
    w = W.WORKLOADS["C5x"]
    inp = W.make_inputs(w)
    dev = to_device(inp)
    a = run_gpu(w, dev)
    b = run_gpu(w, dev)
    assert torch.equal(a, b)
    # [B, N, H, d] storage viewed as [B, H, N, d] (projection output layout).
    devs = {k: v.transpose(1, 2).contiguous().transpose(1, 2) for k, v in dev.items()}
    outs = torch.empty(w.B, w.Nq, w.H, w.d, dtype=a.dtype, device=a.device).transpose(1, 2)
    c = run_gpu(w, devs, out=outs)
    assert torch.equal(a, c)


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_large_logits_stay_finite(dtype):
    w = W.custom(dtype, B=2, H=2, Nq=200, Nk=300, d=64, cfg_id=402)
    inp = W.make_inputs(w, std_qkv=1.0)
    inp["q"] = (inp["q"].float() * 12).to(inp["q"].dtype)
    inp["k"] = (inp["k"].float() * 12).to(inp["k"].dtype)
    out = run_gpu(w, to_device(inp))
    assert torch.isfinite(out).all().item()
    check_full(w, inp, out)


def test_error_status_from_fwd():
    from scaled_dot_product_16_amd import binding
    q = torch.zeros(1, 1, 8, 48, dtype=torch.float16, device="cuda")
    with pytest.raises(binding.AttnError) as e:
        binding.fwd(q, q.clone(), q.clone())
    assert e.value.status == 4  # head dim 48 is not built
