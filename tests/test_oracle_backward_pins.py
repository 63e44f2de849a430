"""Pins for the oracle's backward pass (CPU only).

The gradients of L = sum(dO * O) are checked against central finite
differences of the oracle's own forward in float64 (a route that shares no
code with the backward formulas: every gradient element is a difference of
two forward evaluations), on tiny cases covering every bias and mask kind,
key grids, resized tables and the image layout; and against torch's
autograd of its float64 scaled_dot_product_attention (a library routine)
where the case reduces to it.  A wrong sign, a missing scale, a transposed
dS, a dropped bias path into dQ or a wrong table bin fails them.
"""

import numpy as np
import pytest
import torch

import oracle as O


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def fd_grad(f, x, h=1e-6):
    """Central differences of the scalar f() with respect to every element of x (in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def check_against_fd(q, k, v, dout, bias, mask, names, image=None, atol=2e-7):
    def loss():
        if image is not None:
            o = O.attention_image(q, k, v, image, bias, mask)
        else:
            o = O.attention(q, k, v, bias, mask)
        return float((o * dout).sum())

    if image is not None:
        res = O.attention_image_backward(q, k, v, dout, image, bias, mask)
    else:
        res = O.attention_backward(q, k, v, dout, bias, mask)
    arrays = {"dq": q, "dk": k, "dv": v}
    if bias is not None and bias.kind == "table":
        arrays["dtable"] = bias.table
    if bias is not None and bias.kind == "relpos":
        arrays["drh"], arrays["drw"] = bias.rh, bias.rw
    for name in names:
        np.testing.assert_allclose(res[name], fd_grad(loss, arrays[name]), rtol=0, atol=atol,
                                   err_msg=name)


def test_plain_cross_attention():
    q, k, v = rnd((2, 2, 3, 4), 1), rnd((2, 2, 5, 4), 2), rnd((2, 2, 5, 4), 3)
    check_against_fd(q, k, v, rnd((2, 2, 3, 4), 4), None, None, ["dq", "dk", "dv"])


@pytest.mark.parametrize("grid", [(2, 2), (2, 3), (3, 2)])
def test_table_bias(grid):
    n = grid[0] * grid[1]
    q, k, v = rnd((2, 2, n, 3), 10), rnd((2, 2, n, 3), 11), rnd((2, 2, n, 3), 12)
    table = rnd(((2 * grid[0] - 1) * (2 * grid[1] - 1), 2), 13)
    bias = O.Bias("table", grid=grid, table=table)
    check_against_fd(q, k, v, rnd((2, 2, n, 3), 14), bias, None, ["dq", "dk", "dv", "dtable"])


@pytest.mark.parametrize("grid,kgrid,nh,nw", [((2, 3), None, None, None), ((3, 2), (2, 4), None, None),
                                            ((2, 3), None, 5, 2), ((2, 2), (3, 2), 2, 7)])
def test_relpos_bias(grid, kgrid, nh, nw):
    kg = kgrid or grid
    nq, nk = grid[0] * grid[1], kg[0] * kg[1]
    d = 3
    q, k, v = rnd((1, 2, nq, d), 20), rnd((1, 2, nk, d), 21), rnd((1, 2, nk, d), 22)
    nh = nh or 2 * max(grid[0], kg[0]) - 1
    nw = nw or 2 * max(grid[1], kg[1]) - 1
    bias = O.Bias("relpos", grid=grid, kgrid=kgrid, rh=rnd((nh, d), 23), rw=rnd((nw, d), 24))
    check_against_fd(q, k, v, rnd((1, 2, nq, d), 25), bias, None, ["dq", "dk", "dv", "drh", "drw"])


def test_relpos_bias_wider_grid_two_batch_items():
    # A 4x6 grid (rows and columns of different lengths) over two batch items
    # and two heads: the table gradients sum over every (b, h, i, kh / kw).
    grid, d = (4, 6), 2
    n = grid[0] * grid[1]
    q, k, v = rnd((2, 2, n, d), 50), rnd((2, 2, n, d), 51), rnd((2, 2, n, d), 52)
    bias = O.Bias("relpos", grid=grid, rh=rnd((7, d), 53), rw=rnd((11, d), 54))
    check_against_fd(q, k, v, rnd((2, 2, n, d), 55), bias, None, ["dq", "dk", "drh", "drw"])


def test_shift_mask_image_layout_with_padding():
    # 5x4 image in 3x3 windows (padded to 6x6), shift 1, table bias, regions.
    window = (5, 4, 3, 3, 1, 1)
    q, k, v = rnd((1, 2, 20, 3), 30), rnd((1, 2, 20, 3), 31), rnd((1, 2, 20, 3), 32)
    bias = O.Bias("table", grid=(3, 3), table=rnd((25, 2), 33))
    mask = O.Mask("shift", window=window)
    check_against_fd(q, k, v, rnd((1, 2, 20, 3), 34), bias, mask, ["dq", "dk", "dv", "dtable"],
                     image=window)


def test_additive_mask_has_no_gradient_path():
    q, k, v = rnd((3, 1, 4, 2), 40), rnd((3, 1, 4, 2), 41), rnd((3, 1, 4, 2), 42)
    mask = O.Mask("additive", add=rnd((2, 4, 4), 43))
    check_against_fd(q, k, v, rnd((3, 1, 4, 2), 44), None, mask, ["dq", "dk", "dv"])


def test_matches_torch_autograd_of_sdpa():
    # Library routine: torch's float64 scaled_dot_product_attention with the
    # table bias as a float attention mask; its mask gradient, summed into
    # the table bins, is the table gradient.
    gh, gw, H, d, B = 3, 3, 2, 4, 2
    n = gh * gw
    q, k, v, do = (rnd((B, H, n, d), s) for s in (50, 51, 52, 53))
    table = rnd(((2 * gh - 1) * (2 * gw - 1), H), 54)
    idx = O.table_relative_index(gh, gw)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    tm = torch.tensor(np.transpose(table[idx], (2, 0, 1))[None].repeat(B, 0), requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm)
    (o * torch.tensor(do)).sum().backward()
    res = O.attention_backward(q, k, v, do, O.Bias("table", grid=(gh, gw), table=table))
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(res[name], t.grad.numpy(), rtol=0, atol=1e-12, err_msg=name)
    dtab = np.zeros_like(table)
    gm = tm.grad.numpy().sum(axis=0)  # [H, n, n]
    for h in range(H):
        np.add.at(dtab[:, h], idx, gm[h])
    np.testing.assert_allclose(res["dtable"], dtab, rtol=0, atol=1e-12)
