"""GPU parity of the 8-bit input path: q, k, v as E4M3 codes with one scale
per tensor (attn_fwd_opt with qkv_format = E4M3), f16/bf16 compute and
output, against the fp64 oracle on the dequantized values, every output
element.

Covers the Swin-T stage-1 shifted windows at full size (image layout,
table bias, region mask), SD self- and cross-attention at full size, every
head dim in both compute dtypes, ragged and multi-tile shapes, table bias,
additive bias and mask, the region mask on the tiled form, padded images,
and strided (8-byte aligned) inputs.  The tolerance is the compute dtype's:
the codes widen exactly, and the scales enter in fp32.
"""

import sys

import pytest
import torch

from scaled_dot_product_16_amd import workloads as W
from tests.helpers import TOL, check_full, check_full_pooled, run_gpu, to_device, with_dense_terms

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from scaled_dot_product_16_amd import binding
    binding.lib()


def test_swin_t_stage1_e4m3_full():
    w = W.WORKLOADS["C2f8"]
    say(f"[e4m3] {w.name} at full size")
    inp = W.make_inputs(w)
    out = run_gpu(w, to_device(inp))
    assert out.dtype == torch.float16
    err = check_full(w, inp, out, name=f"C2f8 {w.name}")
    say(f"  max abs err {err:.3e}")


@pytest.mark.parametrize("key", ["C5xf8", "C5sf8"])
def test_sd_e4m3_full(key):
    w = W.WORKLOADS[key]
    say(f"[e4m3] {w.name} at full size, pooled oracle")
    inp = W.make_inputs(w)
    out = run_gpu(w, to_device(inp))
    res = check_full_pooled(w, inp, out, name=f"{key} {w.name}")
    say(f"  max abs err {res['err']:.3e} over {res['units']} units")


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("d", [32, 40, 64, 80])
@pytest.mark.parametrize("nq,nk", [(49, 49), (64, 1), (1, 17), (130, 77), (300, 1100), (200, 64), (65, 129)])
def test_e4m3_shapes(dtype, d, nq, nk):
    w = W.custom(dtype, B=3, H=2, Nq=nq, Nk=nk, d=d, qkv="e4m3", cfg_id=960 + d)
    say(f"[e4m3] {dtype} d={d} Nq={nq} Nk={nk}")
    inp = W.make_inputs(w, seed=nq * 1000 + nk)
    out = run_gpu(w, to_device(inp))
    assert out.dtype == {W.F16: torch.float16, W.BF16: torch.bfloat16}[dtype]
    check_full(w, inp, out)


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("n,bias,mask", [(49, "additive", "additive"), (300, "additive", "none"),
                                         (200, "none", "additive"), (130, "additive", "additive")])
def test_e4m3_dense_terms(dtype, n, bias, mask):
    w = W.custom(dtype, B=4, H=2, Nq=n, Nk=n, d=64, bias=bias, mask=mask, qkv="e4m3", cfg_id=970)
    say(f"[e4m3] {dtype} N={n} bias={bias} mask={mask}")
    inp = with_dense_terms(w, W.make_inputs(w, seed=n), n_bias=2, n_mask=3)
    check_full(w, inp, run_gpu(w, to_device(inp)))


@pytest.mark.parametrize("geom,grid,d", [((16, 16, 4, 8, 2, 5), (4, 8), 32),
                                         ((15, 13, 7, 7, 3, 3), (7, 7), 40),
                                         ((24, 24, 12, 12, 6, 6), (12, 12), 64),
                                         ((20, 30, 10, 10, 0, 0), (10, 10), 80)])
def test_e4m3_image_layout(geom, grid, d):
    # Windows of up to 64 tokens take the window form, larger ones the tiled
    # form; padded images and shifts on both.
    ih, iw, wh, ww, sh, sw = geom
    nW = (-(-ih // wh)) * (-(-iw // ww))
    mask = "shift" if sh or sw else "none"
    w = W.custom(W.F16, B=2 * nW, H=3, Nq=wh * ww, Nk=wh * ww, d=d, bias="table", grid=grid, mask=mask,
                 layout="image", images=2, window=geom, qkv="e4m3", cfg_id=980)
    say(f"[e4m3] image {geom} d={d}")
    inp = W.make_inputs(w, seed=sum(geom), std_table=0.5)
    check_full(w, inp, run_gpu(w, to_device(inp)))


def test_e4m3_strided_inputs_and_float8_dtype():
    # q, k, v as float8_e4m3fn views of [B, N, H, 48]-wide buffers (rows 8-byte
    # aligned, not 16), d = 40, on the tiled and the two-tile forms.
    from scaled_dot_product_16_amd import binding

    for nk in (300, 77):
        w = W.custom(W.F16, B=2, H=3, Nq=257, Nk=nk, d=40, qkv="e4m3", cfg_id=990)
        say(f"[e4m3] strided float8_e4m3fn views, Nk={nk}")
        inp = W.make_inputs(w, seed=nk)
        dev = to_device(inp)

        def strided(x):
            B_, H_, N_, D_ = x.shape
            buf = torch.zeros(B_, N_, H_, 48, dtype=torch.uint8, device=x.device)
            buf[..., :D_] = x.permute(0, 2, 1, 3)
            return buf.permute(0, 2, 1, 3)[..., :D_].view(torch.float8_e4m3fn)

        q, k, v = (strided(dev[n]) for n in ("q", "k", "v"))
        assert q.stride(2) == 3 * 48
        out = binding.fwd(q, k, v, qkv_descale=tuple(inp["descale"].tolist()))
        torch.cuda.synchronize()
        check_full(w, inp, out)


def test_e4m3_matches_f16_path_on_exact_values():
    # Codes whose scaled values are exact in f16 (power-of-two scales): the
    # 8-bit path and the f16 path see the same numbers and use the same
    # arithmetic, so they agree to the last bit except where the folded
    # q*k scale rounds differently from 1/sqrt(d) (not here: scales 1).
    w = W.custom(W.F16, B=4, H=3, Nq=300, Nk=300, d=64, qkv="e4m3", cfg_id=991)
    inp = W.make_inputs(w)
    dev = to_device(inp)
    from scaled_dot_product_16_amd import binding

    o8 = binding.fwd(dev["q"], dev["k"], dev["v"], qkv_descale=(1.0, 1.0, 1.0))
    f = lambda x: x.view(torch.float8_e4m3fn).to(torch.float16)
    o16 = binding.fwd(f(dev["q"]), f(dev["k"]), f(dev["v"]))
    torch.cuda.synchronize()
    assert torch.equal(o8, o16)
    # And with the test's scales, within the tolerance of the oracle.
    check_full(w, inp, binding.fwd(dev["q"], dev["k"], dev["v"], qkv_descale=tuple(inp["descale"].tolist())))
