"""GPU parity of the backward pass (attn_bwd) against the oracle's fp64
gradients, every element: dQ, dK, dV and the table gradient, for Swin
windows in both layouts (shift, region mask and zero padding folded into
the addressing), every head dim, ragged windows, every bias and mask kind
the window path takes.

Tolerance: the forward's max-abs bound for the dtype (f16 5e-3, bf16 2e-2),
scaled by max(1, max |reference|) of each gradient: gradients are not N(0,1)
(the table gradient sums dS over all windows), the products round dS and P
to the element type, and the outputs are rounded to it (a relative error of
2^-11 / 2^-8 per element).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_16_amd import binding as Bd
from scaled_dot_product_16_amd import workloads as W
from tests.helpers import TOL, oracle_arrays, record, to_device, with_dense_terms

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Bd.lib()


def run_bwd(w, dev):
    kw = W.device_args(w, dev)
    out = Bd.bwd(dev["q"], dev["k"], dev["v"], dev["dout"], **kw)
    torch.cuda.synchronize()
    return out


def check_grads(w, inp, got, name=None):
    arrs = oracle_arrays(inp)
    ref = oracle.run_workload_backward(w, arrs)
    worst = {}
    pairs = list(zip(("dq", "dk", "dv"), got[:3]))
    if w.bias == "relpos":
        pairs += [("drh", got[3][0]), ("drw", got[3][1])]
    elif w.bias == "table":
        pairs += [("dtable", got[3])]
    else:
        assert got[3] is None
    for key, g in pairs:
        r = ref[key]
        gg = g.detach().to("cpu", torch.float64).numpy()
        assert np.all(np.isfinite(gg)), key
        err = float(np.max(np.abs(gg - r)))
        tol = TOL[w.dtype] * max(1.0, float(np.max(np.abs(r))))
        worst[key] = err
        if name:
            record(f"{name} {key}", w.dtype, err, tol, gg.size)
        assert err <= tol, f"{key}: max abs err {err:.3e} > {tol:.3e}"
    return worst


def inputs(w, seed=0, std_table=0.5):
    inp = W.make_inputs(w, seed=seed, std_table=std_table)
    inp["dout"] = W.to_dtype(W.normal(w.q_shape, w.cfg_id, 7, 1.0, seed), w.dtype)
    return inp


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_swin_t_stage1_backward(dtype):
    # The Swin-T stage-1 shifted-window workload at full size (image layout,
    # table bias, region mask).
    base = W.WORKLOADS["C2"]
    w = W.custom(dtype, B=base.B, H=base.H, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7),
                 mask="shift", layout="image", images=8, window=base.window, cfg_id=base.cfg_id)
    say(f"[backward] Swin-T stage 1 at full size, {dtype}")
    inp = inputs(w, std_table=0.02)
    worst = check_grads(w, inp, run_bwd(w, to_device(inp)), name=f"backward C2 shape {dtype}")
    say(f"  max abs errors {worst}")


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("d", [32, 40, 64, 80])
@pytest.mark.parametrize("nq,nk", [(49, 49), (64, 64), (7, 64), (64, 1), (33, 50)])
def test_backward_shapes(dtype, d, nq, nk):
    w = W.custom(dtype, B=3, H=2, Nq=nq, Nk=nk, d=d, cfg_id=800 + d)
    say(f"[backward] {dtype} d={d} Nq={nq} Nk={nk}")
    inp = inputs(w, seed=nq * 100 + nk)
    check_grads(w, inp, run_bwd(w, to_device(inp)))


CASES = [
    ("table", (7, 7), "none", None),
    ("table", (8, 8), "none", None),
    ("table", (4, 9), "none", None),
    ("none", None, "shift", (16, 16, 4, 8, 2, 5)),
    ("table", (7, 7), "shift", (28, 21, 7, 7, 3, 2)),
    ("additive", None, "none", None),
    ("none", None, "additive", None),
    ("table", (7, 7), "additive", None),
    ("additive", None, "shift", (14, 14, 7, 7, 3, 3)),
    # Extreme window shapes for the table gradient's two stages: 16 x 4,
    # 64 x 1 (the largest intermediate, 64 * 64 sums) and 1 x 64.
    ("table", (16, 4), "none", None),
    ("table", (64, 1), "none", None),
    ("table", (1, 64), "none", None),
]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_bias_and_mask(dtype, case):
    bias, grid, mask, window = CASES[case]
    if mask == "shift":
        ih, iw, wh, ww = window[:4]
        n, B = wh * ww, 2 * (ih // wh) * (iw // ww)
    else:
        n, B = (grid[0] * grid[1] if grid else 60), 6
    w = W.custom(dtype, B=B, H=3, Nq=n, Nk=n, d=32, bias=bias, grid=grid, mask=mask, window=window,
                 cfg_id=820 + case)
    say(f"[backward] {dtype} {bias} {grid} {mask} {window}")
    inp = with_dense_terms(w, inputs(w, seed=case), n_bias=2, n_mask=3)
    check_grads(w, inp, run_bwd(w, to_device(inp)))


@pytest.mark.parametrize("d", [40, 64, 80])
def test_backward_table_head_dims(d):
    # The fp32 dS^T of the table gradient in the dead K / V tiles (which
    # hold it at every head dim above 32; at d = 32 an 8 x 8 window needs
    # its own region, covered above).
    w = W.custom(W.BF16, B=6, H=3, Nq=64, Nk=64, d=d, bias="table", grid=(8, 8), cfg_id=830 + d)
    say(f"[backward] table bias 8x8, d={d}")
    inp = inputs(w, seed=d)
    check_grads(w, inp, run_bwd(w, to_device(inp)))


@pytest.mark.parametrize("geom", [(15, 13, 7, 7, 3, 3), (20, 25, 4, 8, 2, 5), (14, 14, 7, 7, 0, 0)])
def test_backward_padded_image_layout(geom):
    ih, iw, wh, ww, sh, sw = geom
    ph, pw = -(-ih // wh) * wh, -(-iw // ww) * ww
    nW = (ph // wh) * (pw // ww)
    mask = "shift" if sh or sw else "none"
    w = W.custom(W.F16, B=2 * nW, H=3, Nq=wh * ww, Nk=wh * ww, d=32, bias="table", grid=(wh, ww),
                 mask=mask, layout="image", images=2, window=geom, cfg_id=840)
    say(f"[backward] padded image {geom}")
    inp = inputs(w, seed=sum(geom))
    check_grads(w, inp, run_bwd(w, to_device(inp)))


def test_backward_deterministic_and_strided():
    w = W.custom(W.BF16, B=64, H=3, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7), cfg_id=850)
    say("[backward] determinism and [B, N, H, d] strides")
    inp = inputs(w, seed=5)
    dev = to_device(inp)
    a = run_bwd(w, dev)
    b = run_bwd(w, dev)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # The same call on [B, N, H, d] storage viewed as [B, H, N, d].
    devs = {k: (v.transpose(1, 2).contiguous().transpose(1, 2) if k in ("q", "k", "v", "dout") else v)
            for k, v in dev.items()}
    outs = [torch.empty(w.B, w.Nq, w.H, w.d, dtype=dev["q"].dtype, device="cuda").transpose(1, 2)
            for _ in range(3)]
    kw = W.device_args(w, devs)
    c = Bd.bwd(devs["q"], devs["k"], devs["v"], devs["dout"], dq=outs[0], dk=outs[1], dv=outs[2], **kw)
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("d", [32, 40, 64, 80])
@pytest.mark.parametrize("nq,nk", [(65, 65), (200, 300), (300, 77), (129, 1000), (1, 130)])
def test_tiled_backward_shapes(dtype, d, nq, nk):
    # Longer than one window: the row kernel (log-sum-exp, D, dQ) and the
    # column kernel (dK, dV), ragged query and key tiles.
    w = W.custom(dtype, B=2, H=2, Nq=nq, Nk=nk, d=d, cfg_id=870 + d)
    say(f"[tiled backward] {dtype} d={d} Nq={nq} Nk={nk}")
    inp = inputs(w, seed=nq + nk)
    check_grads(w, inp, run_bwd(w, to_device(inp)), name=f"tiled backward {nq}x{nk} d={d}")


@pytest.mark.parametrize("key", ["C5s", "C5x"])
def test_tiled_backward_sd_shapes(key):
    # SD UNet self- and cross-attention shapes, every element compared on a
    # slice of 2 batch items (the oracle's gradient is per (b, h) anyway).
    base = W.WORKLOADS[key]
    w = W.custom(base.dtype, B=2, H=base.H, Nq=base.Nq, Nk=base.Nk, d=base.d, cfg_id=base.cfg_id)
    say(f"[tiled backward] {key} shape, 2 of {base.B} batch items")
    inp = inputs(w, seed=1)
    check_grads(w, inp, run_bwd(w, to_device(inp)), name=f"tiled backward {key} shape (2 batch items)")


def test_backward_unsupported_calls():
    w = W.custom(W.F16, B=1, H=2, Nq=100, Nk=64, d=64, bias="relpos", grid=(10, 10), kgrid=(8, 8),
                 cfg_id=880)
    dev = to_device(inputs(w))
    with pytest.raises(Bd.AttnError) as e:                # relative position with a key grid
        Bd.bwd(dev["q"], dev["k"], dev["v"], dev["dout"], **W.device_args(w, dev))
    assert e.value.status == 4
    q = torch.zeros(1, 2, 49, 32, dtype=torch.float32, device="cuda")
    with pytest.raises(Bd.AttnError) as e:
        Bd.bwd(q, q.clone(), q.clone(), q.clone())       # fp32
    assert e.value.status == 4


# Relative-position backward (tiled path): equal grids, tables of 2g-1 rows.
# gh + gw <= 32 with at most 256 keys: the one-hot table form ((16, 16) and
# (17, 15) at its limits); (16, 17), (30, 30): the general form; gw = 64:
# the 64-wide form.
RELPOS_GRIDS = [(2, 3), (7, 7), (14, 14), (8, 12), (5, 16), (16, 16), (17, 15), (16, 17), (30, 30),
                (1, 64), (3, 64), (16, 64)]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("grid", RELPOS_GRIDS)
def test_relpos_backward_grids(dtype, grid):
    n = grid[0] * grid[1]
    w = W.custom(dtype, B=2, H=3, Nq=n, Nk=n, d=64, bias="relpos", grid=grid, cfg_id=860)
    say(f"[backward] relpos {dtype} grid {grid}")
    inp = inputs(w, seed=n, std_table=0.5)
    check_grads(w, inp, run_bwd(w, to_device(inp)))


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("d", [32, 40, 64, 80])
@pytest.mark.parametrize("grid", [(14, 14), (12, 24), (4, 64)])
def test_relpos_backward_head_dims(dtype, d, grid):
    n = grid[0] * grid[1]
    w = W.custom(dtype, B=2, H=2, Nq=n, Nk=n, d=d, bias="relpos", grid=grid, cfg_id=870 + d)
    say(f"[backward] relpos {dtype} d={d} grid {grid}")
    inp = inputs(w, seed=d, std_table=0.5)
    check_grads(w, inp, run_bwd(w, to_device(inp)))


def test_relpos_backward_sam_windows():
    # SAM ViT-B windowed attention: 25 windows of 14x14 (one 64x64 image
    # padded to 70x70), 12 heads, d=64, bf16, tables at the workload's
    # N(0, 0.02^2).
    w = W.custom(W.BF16, B=25, H=12, Nq=196, Nk=196, d=64, bias="relpos", grid=(14, 14), cfg_id=3)
    say("[backward] SAM-B windowed, one image")
    inp = inputs(w, std_table=0.02)
    worst = check_grads(w, inp, run_bwd(w, to_device(inp)), name="relpos backward SAM-B windows")
    say(f"  max abs errors {worst}")


@pytest.mark.parametrize("d,heads", [(64, 2), (80, 2)])
def test_relpos_backward_sam_global(d, heads):
    # SAM global attention: the 64x64 grid at full length (4096 tokens),
    # one image and two heads (the oracle's fp64 backward of a 4096-token
    # unit takes a few seconds).
    w = W.custom(W.BF16, B=1, H=heads, Nq=4096, Nk=4096, d=d, bias="relpos", grid=(64, 64),
                 cfg_id=4 if d == 64 else 44)
    say(f"[backward] SAM global 64x64, d={d}")
    inp = inputs(w, std_table=0.02)
    worst = check_grads(w, inp, run_bwd(w, to_device(inp)), name=f"relpos backward SAM global d={d}")
    say(f"  max abs errors {worst}")


def test_relpos_backward_one_hot_form_deterministic():
    # SAM-style 14 x 14 windows take the one-hot key table form (bias and
    # dRh/dRw gathers as matrix products, a fixed-order partial reduction):
    # two calls agree bitwise, and the result matches the oracle.
    w = W.custom(W.BF16, B=6, H=3, Nq=196, Nk=196, d=64, bias="relpos", grid=(14, 14), cfg_id=895)
    inp = inputs(w, seed=5, std_table=0.5)
    dev = to_device(inp)
    a = run_bwd(w, dev)
    b = run_bwd(w, dev)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert torch.equal(a[3][0], b[3][0]) and torch.equal(a[3][1], b[3][1])
    check_grads(w, inp, a)


def test_relpos_backward_bias_is_seen_and_deterministic():
    # The table gradients and the bias path into dQ are large next to the
    # tolerance with tables of std 0.5; two calls agree bitwise.
    w = W.custom(W.BF16, B=2, H=2, Nq=128 * 2, Nk=128 * 2, d=64, bias="relpos", grid=(4, 64),
                 cfg_id=890)
    inp = inputs(w, seed=3, std_table=0.5)
    dev = to_device(inp)
    a = run_bwd(w, dev)
    b = run_bwd(w, dev)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert torch.equal(a[3][0], b[3][0]) and torch.equal(a[3][1], b[3][1])
    ref = oracle.run_workload_backward(w, oracle_arrays(inp))
    plain = oracle.run_workload_backward(
        W.custom(W.BF16, B=2, H=2, Nq=256, Nk=256, d=64, cfg_id=890), oracle_arrays(inp))
    # The bias changes dq by far more than the tolerance.
    assert np.max(np.abs(ref["dq"] - plain["dq"])) > 10 * TOL[W.BF16]
    assert np.max(np.abs(ref["drh"])) > 10 * TOL[W.BF16]
