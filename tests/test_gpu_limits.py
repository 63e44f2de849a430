"""GPU parity at the size limits of the on-chip index data, and the
rejection of a call whose index data does not fit.

* the largest relative-position table the TABLE bias accepts: a 64 x 64
  grid has (2*64-1)^2 = 16129 table rows (the limit is 16384), held in LDS
  next to the per-key index data of 4096 keys;
* the decomposed relative position in its table form on a large grid that
  is neither 64 wide nor small enough for the contraction form (56 x 56:
  per-query relh/relw rows for 112 offsets in LDS);
* a 100 x 100 grid, whose per-query tables do not fit in LDS: the call
  returns E_UNSUPPORTED and launches nothing.
Rows are sampled across tile boundaries and compared with the fp64 oracle.
"""

import sys

import pytest
import torch

from scaled_dot_product_16_amd import binding as Bnd
from scaled_dot_product_16_amd import workloads as W
from tests.helpers import TOL, check_sampled, run_gpu, sample_select, to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Bnd.lib()


@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.F32])
def test_largest_table_bias(dtype):
    w = W.custom(dtype, B=1, H=2, Nq=4096, Nk=4096, d=32, bias="table", grid=(64, 64), cfg_id=700)
    say(f"[limits] table bias on a 64x64 grid, {dtype}")
    inp = W.make_inputs(w, seed=1)
    out = run_gpu(w, to_device(inp))
    err = check_sampled(w, inp, out, sample_select(w, n_pairs=2, n_rows=48))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]:.0e})")


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_relpos_table_form_large_grid(dtype):
    w = W.custom(dtype, B=1, H=2, Nq=3136, Nk=3136, d=64, bias="relpos", grid=(56, 56), cfg_id=701)
    say(f"[limits] relpos on a 56x56 grid (table form), {dtype}")
    inp = W.make_inputs(w, seed=2)
    out = run_gpu(w, to_device(inp))
    err = check_sampled(w, inp, out, sample_select(w, n_pairs=2, n_rows=48))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]:.0e})")


def test_index_data_too_large_is_rejected():
    w = W.custom(W.BF16, B=1, H=1, Nq=10000, Nk=10000, d=64, bias="relpos", grid=(100, 100), cfg_id=702)
    say("[limits] relpos on a 100x100 grid: E_UNSUPPORTED, nothing launched")
    dev = to_device(W.make_inputs(w, seed=3))
    # The host validation already knows: attn_check gives the status attn_fwd returns.
    assert Bnd.check(dev["q"], dev["k"], dev["v"], **W.device_args(w, dev)) == 4
    with pytest.raises(Bnd.AttnError) as e:
        Bnd.fwd(dev["q"], dev["k"], dev["v"], **W.device_args(w, dev))
    assert e.value.status == 4
    torch.cuda.synchronize()


def test_empty_query_set_and_empty_key_set():
    # Zero query rows: an empty output and no launch.  Zero keys with queries
    # present: rejected (a softmax over no keys is undefined).
    q = torch.zeros(2, 3, 0, 64, dtype=torch.float16, device="cuda")
    k = torch.randn(2, 3, 10, 64, dtype=torch.float16, device="cuda")
    out = Bnd.fwd(q, k, k.clone())
    assert out.shape == (2, 3, 0, 64)
    q = torch.randn(2, 3, 5, 64, dtype=torch.float16, device="cuda")
    k = torch.zeros(2, 3, 0, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(Bnd.AttnError):
        Bnd.fwd(q, k, k.clone())
    torch.cuda.synchronize()
