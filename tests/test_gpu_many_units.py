"""GPU parity at large work-unit counts against the fp64 oracle.

The MFMA kernels split each (batch, head) into query tiles of 128 rows; the
shapes here have thousands of such units, more than the device holds at
once, with ragged query tiles, key counts around two key tiles (Nk = 77,
128, 129), and the relative-position bias folded into the contraction, in
the batched and in the windowed image layout.  Every output element is
compared with the oracle.
"""

import sys

import pytest

from scaled_dot_product_16_amd import workloads as W
from tests.helpers import TOL, check_full, run_gpu, to_device

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


# (dtype, head dim, Nk): 24 x 8 heads x 8 query tiles (Nq = 1000, the last
# tile ragged) = 1536 units.
PLAIN = [
    (W.F16, 40, 77),    # cross-attention shape
    (W.BF16, 40, 128),  # exactly two full key tiles
    (W.F16, 64, 129),   # one key into a third tile
    (W.BF16, 64, 1),
    (W.F16, 80, 100),
    (W.BF16, 80, 300),
]


@pytest.mark.parametrize("case", range(len(PLAIN)))
def test_many_units_plain(case):
    dtype, d, nk = PLAIN[case]
    w = W.custom(dtype, B=24, H=8, Nq=1000, Nk=nk, d=d, cfg_id=500 + case)
    say(f"[many units plain] {dtype} d={d} B=24 H=8 Nq=1000 Nk={nk}")
    inp = W.make_inputs(w, seed=case)
    err = check_full(w, inp, run_gpu(w, to_device(inp)))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]:.0e})")


# Relative position folded into the contraction (gh + gw <= 32).
RELPOS = [
    # (dtype, head dim, grid, batch, heads)
    (W.BF16, 64, (14, 14), 300, 4),  # 2 query tiles per head, 2400 units
    (W.F16, 64, (8, 20), 400, 3),    # 160 tokens: second query tile holds 32
    (W.BF16, 40, (10, 12), 600, 2),  # one query tile per head
    (W.F16, 32, (5, 27), 500, 3),    # wide, short grid (gw close to the limit)
]


@pytest.mark.parametrize("case", range(len(RELPOS)))
def test_many_units_relpos(case):
    dtype, d, grid, B, H = RELPOS[case]
    n = grid[0] * grid[1]
    w = W.custom(dtype, B=B, H=H, Nq=n, Nk=n, d=d, bias="relpos", grid=grid, cfg_id=520 + case)
    say(f"[many units relpos] {dtype} d={d} grid={grid} B={B} H={H}")
    inp = W.make_inputs(w, seed=case)
    err = check_full(w, inp, run_gpu(w, to_device(inp)))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]:.0e})")


@pytest.mark.parametrize("bias", ["none", "relpos"])
def test_many_units_image_layout(bias):
    # 16 images of 48 x 48 tokens in 12 x 12 windows: 256 windows of 144
    # tokens, 4 heads, 2 query tiles each -> 2048 units.
    geom = (48, 48, 12, 12, 0, 0)
    nW = 16
    w = W.custom(W.BF16, B=16 * nW, H=4, Nq=144, Nk=144, d=64, bias=bias,
                 grid=(12, 12) if bias == "relpos" else None, layout="image", images=16,
                 window=geom, cfg_id=540)
    say(f"[many units image] bias={bias} {geom}")
    inp = W.make_inputs(w, seed=7)
    err = check_full(w, inp, run_gpu(w, to_device(inp)))
    say(f"  max abs err {err:.3e} (tol {TOL[W.BF16]:.0e})")
