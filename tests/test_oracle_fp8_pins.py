"""Pins of the oracle's 8-bit input path (CPU only).

``e4m3_decode`` follows the E4M3 format of the OCP 8-bit floating point
specification (sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals,
no infinities, S.1111.111 = NaN).  It is pinned against torch's own
float8_e4m3fn conversion on every code (an independent implementation of the
same format) and against values the format fixes in closed form.  The
workload path (codes + one scale per tensor -> attention) is pinned against
torch's scaled_dot_product_attention in float64 on inputs that torch
decodes itself, and by the linearity the scales must have.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_16_amd import workloads as W


def torch_decode(codes) -> np.ndarray:
    t = torch.as_tensor(np.asarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_on_every_code():
    codes = np.arange(256)
    ours, ref = oracle.e4m3_decode(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_decode_closed_forms(code, value):
    assert oracle.e4m3_decode([code])[0] == value


def test_decode_special_codes_and_order():
    v = oracle.e4m3_decode(np.arange(256))
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    # Magnitudes rise strictly with the code; the sign bit only flips the sign.
    assert np.all(np.diff(v[:0x7F]) > 0)
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    assert np.nanmax(np.abs(v)) == 448.0


def test_decode_rejects_non_bytes():
    with pytest.raises(ValueError):
        oracle.e4m3_decode([256])
    with pytest.raises(ValueError):
        oracle.e4m3_decode([-1])


def test_dequantize_is_code_times_scale():
    codes = np.arange(0, 127)
    assert np.array_equal(oracle.dequantize_e4m3(codes, 0.375), 0.375 * torch_decode(codes))


def _sdpa(q, k, v):
    f = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(f(q), f(k), f(v)).numpy()


@pytest.mark.parametrize("nq,nk,d", [(49, 49, 32), (70, 13, 40)])
def test_fp8_workload_matches_sdpa(nq, nk, d):
    w = W.custom(W.F16, B=2, H=3, Nq=nq, Nk=nk, d=d, qkv="e4m3", cfg_id=950)
    inp = W.make_inputs(w, seed=nq)
    s = inp["descale"].numpy().astype(np.float64)
    arrays = {k: v.numpy() for k, v in inp.items()}
    got = oracle.run_workload(w, arrays)
    ref = _sdpa(s[0] * torch_decode(arrays["q"]), s[1] * torch_decode(arrays["k"]),
                s[2] * torch_decode(arrays["v"]))
    assert np.max(np.abs(got - ref)) < 1e-12
    # The three scales are distinct, so a scale applied to the wrong tensor
    # would change the result.
    assert len(set(s.tolist())) == 3


def test_fp8_scales_enter_as_they_must():
    w = W.custom(W.F16, B=1, H=2, Nq=33, Nk=21, d=32, qkv="e4m3", cfg_id=951)
    inp = W.make_inputs(w)
    arrays = {k: v.numpy() for k, v in inp.items()}
    base = oracle.run_workload(w, arrays)
    s = arrays["descale"].astype(np.float64)
    # The value scale is linear in the output.
    o2 = oracle.run_workload(w, dict(arrays, descale=s * [1, 1, 2]))
    assert np.allclose(o2, 2 * base, rtol=1e-13, atol=1e-13)
    # Query and key scales only enter through their product.
    o3 = oracle.run_workload(w, dict(arrays, descale=s * [4, 0.25, 1]))
    assert np.allclose(o3, base, rtol=1e-12, atol=1e-12)
    # ... which does change the result.
    o4 = oracle.run_workload(w, dict(arrays, descale=s * [4, 1, 1]))
    assert np.max(np.abs(o4 - base)) > 1e-2


def test_fp8_image_layout_equals_dequantized_inputs():
    # Swin-T-like shifted windows with a table bias, inputs as codes.
    geom = (14, 14, 7, 7, 3, 3)
    w8 = W.custom(W.F16, B=2 * 4, H=2, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7), mask="shift",
                  layout="image", images=2, window=geom, qkv="e4m3", cfg_id=952)
    inp = W.make_inputs(w8, std_table=0.5)
    arrays = {k: v.numpy() for k, v in inp.items()}
    got = oracle.run_workload(w8, arrays)
    s = arrays["descale"].astype(np.float64)
    w16 = W.custom(W.F16, B=2 * 4, H=2, Nq=49, Nk=49, d=32, bias="table", grid=(7, 7), mask="shift",
                   layout="image", images=2, window=geom, cfg_id=952)
    plain = dict(arrays, q=s[0] * torch_decode(arrays["q"]), k=s[1] * torch_decode(arrays["k"]),
                 v=s[2] * torch_decode(arrays["v"]), table=arrays["table"].astype(np.float64))
    ref = oracle.run_workload(w16, plain)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_input_generator_scales_and_codes():
    w = W.custom(W.F16, B=3, H=2, Nq=40, Nk=40, d=64, qkv="e4m3", cfg_id=953)
    inp = W.make_inputs(w)
    for i, name in enumerate(("q", "k", "v")):
        codes = inp[name].numpy()
        assert codes.dtype == np.uint8
        vals = torch_decode(codes)
        # Scale = max|x| / 448: the largest code decodes to 448 in magnitude.
        assert np.max(np.abs(vals)) == 448.0
        assert not np.any(np.isnan(vals))
        x = W.normal(w.q_shape if name == "q" else w.kv_shape, w.cfg_id, i)
        s = float(inp["descale"][i])
        assert abs(s - float(np.abs(x).max()) / 448.0) <= 1e-7 * s
        # Round to nearest: within half an E4M3 step (2^-4 relative, or
        # 2^-10 absolute in the subnormal range) of x / s.
        err = np.abs(vals - x.astype(np.float64) / s)
        assert np.all(err <= np.maximum(np.abs(x / s) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


def test_pool_dequantizes_like_the_serial_oracle():
    from oracle import pool

    w = W.custom(W.F16, B=2, H=2, Nq=49, Nk=49, d=32, qkv="e4m3", cfg_id=954)
    inp = W.make_inputs(w)
    arrays = {k: v.numpy() for k, v in inp.items()}
    ref = oracle.run_workload(w, arrays)
    with pool.UnitPool(dict(inp, out=torch.from_numpy(ref)), pool.spec_of(w), workers=2) as P:
        res = P.compare(pool.units_of(w))
    assert len(res) == 4 and max(r["err"] for r in res) < 1e-12
