"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and attn_check returns the documented status for each argument error (no GPU
work is issued; attn_check never touches the device)."""

import ctypes
import os
import re

import pytest
import torch

from scaled_dot_product_16_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from scaled_dot_product_16_amd.build import build
        build()
    return B.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    return re.findall(r"ATTN_API\s+[\w\s\*]+?\b(attn_\w+)\s*\(", src)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"attn_fwd", "attn_check", "attn_strerror", "attn_version",
                          "attn_fwd_opt", "attn_check_opt", "attn_bwd", "attn_bwd_opt", "attn_bwd_check",
                          "attn_bwd_workspace_size", "attn_bwd_noalloc"}
    for n in names:
        assert hasattr(lib, n)
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_struct_layout_matches_header(lib):
    # The binding's structs must match the C layout (sizes on x86-64).
    assert ctypes.sizeof(B.AttnTensorC) == 8 + 32 + 24 + 8
    assert ctypes.sizeof(B.WindowC) == 24
    assert ctypes.sizeof(B.BiasDescC) == 4 * 3 + 4 + 8 * 4 + 8 + 16 + 8 + 8
    assert ctypes.sizeof(B.MaskDescC) == 8 + 8 + 8 + 16 + 24 + 4 + 4
    assert ctypes.sizeof(B.OptionsC) == 32
    assert [B.OptionsC.__dict__[f].offset for f in ("window_heads", "qkv_format", "q_descale",
                                                   "k_descale", "v_descale", "reserved", "lse")] == \
        [0, 4, 8, 12, 16, 20, 24]
    assert ctypes.sizeof(B.BwdOptionsC) == 32


def test_strerror_and_version(lib):
    for st in range(8):
        assert lib.attn_strerror(st)
    assert lib.attn_strerror(99) == b"unknown status"
    assert lib.attn_version() >> 16 == 1 and lib.attn_version() & 0xFFFF >= 5


def t(*shape, dtype=torch.float16):
    return torch.zeros(*shape, dtype=dtype)


def test_valid_calls_pass(lib):
    q = t(2, 3, 49, 32)
    assert B.check(q, t(2, 3, 49, 32), t(2, 3, 49, 32)) == 0
    assert B.check(t(1, 1, 5, 40), t(1, 1, 77, 40), t(1, 1, 77, 40)) == 0
    assert B.check(t(1, 1, 5, 12, dtype=torch.float32), t(1, 1, 7, 12, dtype=torch.float32),
                   t(1, 1, 7, 12, dtype=torch.float32)) == 0
    tb = B.TableBias(t(169, 3), (7, 7))
    assert B.check(q, t(2, 3, 49, 32), t(2, 3, 49, 32), bias=tb) == 0
    win = B.Window(56, 56, 7, 7, 3, 3)
    qi = t(8, 3, 3136, 32)
    assert B.check(qi, t(8, 3, 3136, 32), t(8, 3, 3136, 32), bias=tb, mask=B.ShiftMask(win),
                   layout="image") == 0
    rp = B.RelposBias(t(127, 64, dtype=torch.bfloat16), t(127, 64, dtype=torch.bfloat16), (64, 64))
    qb = t(1, 2, 4096, 64, dtype=torch.bfloat16)
    assert B.check(qb, qb.clone(), qb.clone(), bias=rp) == 0


def test_shape_errors(lib):
    q = t(2, 3, 49, 32)
    assert B.check(q, t(1, 3, 49, 32), t(1, 3, 49, 32)) == 2            # batch mismatch
    assert B.check(q, t(2, 2, 49, 32), t(2, 2, 49, 32)) == 2            # heads mismatch
    assert B.check(q, t(2, 3, 49, 32), t(2, 3, 48, 32)) == 2            # k/v length mismatch
    assert B.check(q, t(2, 3, 49, 32), t(2, 3, 49, 32), out=t(2, 3, 48, 32)) == 2
    tb = B.TableBias(t(143, 3), (7, 6))                                  # grid != N
    assert B.check(q, t(2, 3, 49, 32), t(2, 3, 49, 32), bias=tb) == 2
    win = B.Window(56, 56, 7, 7, 3, 3)
    assert B.check(t(8, 3, 3000, 32), t(8, 3, 3000, 32), t(8, 3, 3000, 32), mask=B.ShiftMask(win),
                   layout="image") == 2                                  # image size
    bad = B.Window(56, 56, 7, 7, 7, 0)                                   # shift >= window
    assert B.check(q, t(2, 3, 49, 32), t(2, 3, 49, 32), mask=B.ShiftMask(bad)) == 2
    # An image that is not a whole number of windows is padded to one
    # (50 -> 56 rows here), so it is accepted; its token count must still be
    # img_h * img_w, and batched windows must still hold win_h * win_w tokens.
    nondiv = B.Window(50, 56, 7, 7, 3, 3)
    assert B.check(t(8, 3, 2800, 32), t(8, 3, 2800, 32), t(8, 3, 2800, 32),
                   mask=B.ShiftMask(nondiv), layout="image") == 0
    assert B.check(t(8, 3, 2801, 32), t(8, 3, 2801, 32), t(8, 3, 2801, 32),
                   mask=B.ShiftMask(nondiv), layout="image") == 2
    assert B.check(t(8, 3, 50, 32), t(8, 3, 50, 32), t(8, 3, 50, 32), mask=B.ShiftMask(nondiv)) == 2


def test_empty_tensors_are_rejected(lib):
    # The library takes non-empty tensors only: an empty torch tensor has no
    # storage (NULL data, E_NULL); a zero dimension with a valid pointer is
    # E_SHAPE.  (binding.fwd returns an empty output for zero query rows
    # without calling the library.)
    e = t(0, 3, 49, 32)
    assert B.check(e, e.clone(), e.clone()) == 1
    q = t(2, 3, 49, 32)
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(q, q.clone(), q.clone(), q.clone(), None, None,
                                                   "batched", None)
    qc.dims[2] = 0
    h = B.lib()
    assert h.attn_check(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                        ctypes.byref(md), ctypes.byref(oc), dt) == 2
    del keep


def test_unsupported_and_layout_errors(lib):
    assert B.check(t(1, 1, 8, 48), t(1, 1, 8, 48), t(1, 1, 8, 48)) == 4  # d=48 not built
    assert B.check(t(1, 1, 8, 132, dtype=torch.float32), t(1, 1, 8, 132, dtype=torch.float32),
                   t(1, 1, 8, 132, dtype=torch.float32)) == 4
    base = t(1, 1, 9, 40)
    odd = torch.zeros(1, 1, 9 * 44, dtype=torch.float16)[..., :9 * 44].view(1, 1, 9, 44)[..., :40]
    assert odd.stride(2) == 44
    assert B.check(odd, base, base.clone()) == 3                          # row stride not 16 B
    mis = torch.zeros(1 * 1 * 9 * 40 + 1, dtype=torch.float16)[1:].view(1, 1, 9, 40)
    assert B.check(mis, base, base.clone()) == 3                          # misaligned base
    big = B.RelposBias(t(399, 64), t(399, 64), (200, 200))               # 40000 tokens
    q = t(1, 1, 40000, 64)
    assert B.check(q, q.clone(), q.clone(), bias=big) == 4


def test_alias_and_null_errors(lib):
    q = t(1, 2, 16, 32)
    k, v = t(1, 2, 16, 32), t(1, 2, 16, 32)
    assert B.check(q, k, v, out=q) == 5
    assert B.check(q, k, v, out=v[:, :1].expand(1, 2, 16, 32)) == 5
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(q, k, v, t(1, 2, 16, 32), None, None, "batched", None)
    qc.data = None
    h = B.lib()
    assert h.attn_check(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                        ctypes.byref(md), ctypes.byref(oc), dt) == 1
    assert h.attn_check(None, ctypes.byref(kc), ctypes.byref(vc), None, None, ctypes.byref(oc), dt) == 1
    # Table bias without a table pointer.
    qc.data = q.data_ptr()
    bd.kind, bd.grid_h, bd.grid_w, bd.table = 1, 4, 4, None
    assert h.attn_check(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                        ctypes.byref(md), ctypes.byref(oc), dt) == 1


def test_invalid_enums(lib):
    q = t(1, 2, 16, 32)
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(q, t(1, 2, 16, 32), t(1, 2, 16, 32), t(1, 2, 16, 32),
                                                  None, None, "batched", None)
    h = B.lib()
    args = lambda: (ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                    ctypes.byref(md), ctypes.byref(oc))
    assert h.attn_check(*args(), 3) == 7
    bd.kind = 9
    assert h.attn_check(*args(), dt) == 7
    bd.kind, md.kind = 0, 5
    assert h.attn_check(*args(), dt) == 7
    md.kind = 0
    qc.layout = 4
    assert h.attn_check(*args(), dt) == 7


def test_key_grid_validation(lib):
    bf = torch.bfloat16
    rp = lambda nh, nw, kg: B.RelposBias(t(nh, 64, dtype=bf), t(nw, 64, dtype=bf), (8, 8), kg)
    q = t(1, 2, 64, 64, dtype=bf)
    k = t(1, 2, 256, 64, dtype=bf)
    assert B.check(q, k, k.clone(), bias=rp(31, 31, (16, 16))) == 0
    assert B.check(q, q.clone(), q.clone(), bias=rp(31, 31, (16, 16))) == 2  # Nk != key grid
    k2 = t(1, 2, 32, 64, dtype=bf)
    assert B.check(q, k2, k2.clone(), bias=rp(15, 15, (4, 8))) == 0
    # Tables of another length than 2*max-1 are resized by the kernel.
    assert B.check(q, k, k.clone(), bias=rp(15, 15, (16, 16))) == 0
    with pytest.raises(ValueError):                                         # 1 to 1023 rows
        B.check(q, k, k.clone(), bias=rp(1024, 15, (16, 16)))
    # A 2 x 128 key grid is a valid call whose per-query tables (130 rows)
    # and 255-row prologue scratch do not fit one CU's LDS next to the K/V
    # tiles: E_UNSUPPORTED from the host validation, as from attn_fwd.
    assert B.check(q, k, k.clone(), bias=B.RelposBias(t(15, 64, dtype=bf), t(255, 64, dtype=bf),
                                                      (8, 8), (2, 128))) == 4
    # Per-axis table rows above the limit (2 * 200 - 1 each) are unsupported.
    kb = t(1, 2, 200 * 200, 64, dtype=bf)
    assert B.check(q, kb, kb.clone(), bias=B.RelposBias(t(399, 64, dtype=bf), t(399, 64, dtype=bf),
                                                        (8, 8), (200, 200))) == 4
    # A key grid belongs to the relative-position kind and the batched layout
    # only; one positive and one zero side is a shape error.
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(q, k, k.clone(), q.clone(), rp(31, 31, (16, 16)),
                                                  None, "batched", None)
    h = B.lib()
    args = lambda: (ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                    ctypes.byref(md), ctypes.byref(oc), dt)
    assert h.attn_check(*args()) == 0
    bd.kgrid_w = 0
    assert h.attn_check(*args()) == 2
    bd.kgrid_w = 16
    tab = t(15 * 15, 2, dtype=bf)
    bd.kind, bd.table = 1, tab.data_ptr()
    assert h.attn_check(*args()) == 2
    win = B.Window(16, 16, 8, 8, 0, 0)
    qi = t(1, 2, 256, 64, dtype=bf)
    qc, kc, vc, bd, md, oc, dt, keep2 = B._marshal(qi, qi.clone(), qi.clone(), qi.clone(),
                                                   rp(15, 15, None), None, "image", win)
    assert h.attn_check(*args()) == 0
    bd.kgrid_h, bd.kgrid_w = 8, 8
    assert h.attn_check(*args()) == 2
    del keep, keep2


def test_lds_budget_is_part_of_validation(lib):
    # attn_check runs the kernel choice and its LDS arithmetic (no GPU):
    # calls whose tiles and tables fit are OK, the others E_UNSUPPORTED,
    # exactly as attn_fwd returns them.
    bf = torch.bfloat16
    rp = lambda g, d: B.RelposBias(t(2 * g[0] - 1, d, dtype=bf), t(2 * g[1] - 1, d, dtype=bf), g)
    for grid, d, want in [((64, 64), 64, 0), ((64, 64), 80, 0), ((14, 14), 64, 0),
                          ((56, 56), 64, 0), ((100, 100), 64, 4), ((90, 90), 80, 4)]:
        n = grid[0] * grid[1]
        q = t(1, 1, n, d, dtype=bf)
        assert B.check(q, q.clone(), q.clone(), bias=rp(grid, d)) == want, (grid, d)
    # The largest table bias (64 x 64 grid, 16129 rows) fits next to 4096 keys.
    q = t(1, 2, 4096, 32)
    tab = B.TableBias(t(127 * 127, 2), (64, 64))
    assert B.check(q, q.clone(), q.clone(), bias=tab) == 0
    # fp32: its kernel keeps the per-query tables of 64 queries only, so the
    # 100 x 100 grid fits there (about 99 KB).
    q = t(1, 1, 10000, 32, dtype=torch.float32)
    big = B.RelposBias(t(199, 32, dtype=torch.float32), t(199, 32, dtype=torch.float32), (100, 100))
    assert B.check(q, q.clone(), q.clone(), bias=big) == 0


def test_window_heads_option(lib):
    # Heads of one window per workgroup (the packed short-sequence form):
    # 1 to 4 when they divide H, on half-precision windows with table or no
    # bias and region or no mask; refused otherwise, by attn_check_opt as by
    # attn_fwd_opt.  0 (or no options) is the library's choice.
    q = t(2, 12, 49, 32)
    tab = B.TableBias(t(169, 12), (7, 7))
    for hg, want in [(0, 0), (1, 0), (2, 0), (3, 0), (4, 0), (5, 4), (6, 4), (12, 4), (-1, 7)]:
        assert B.check(q, q.clone(), q.clone(), bias=tab, window_heads=hg) == want, hg
    q3 = t(2, 3, 49, 32)
    assert B.check(q3, q3.clone(), q3.clone(), window_heads=2) == 4    # 2 does not divide 3
    assert B.check(q3, q3.clone(), q3.clone(), window_heads=3) == 0
    qf = t(2, 3, 49, 32, dtype=torch.float32)
    assert B.check(qf, qf.clone(), qf.clone(), window_heads=3) == 4    # no fp32 packed form
    qb = t(2, 4, 49, 64, dtype=torch.bfloat16)
    add = B.AdditiveMask(t(1, 49, 49, dtype=torch.bfloat16))
    assert B.check(qb, qb.clone(), qb.clone(), mask=add, window_heads=2) == 4
    assert B.check(qb, qb.clone(), qb.clone(), mask=add, window_heads=1) == 0
    ql = t(1, 4, 300, 64)
    assert B.check(ql, ql.clone(), ql.clone(), window_heads=2) == 4    # not a window-sized call
    assert B.check(ql, ql.clone(), ql.clone(), window_heads=1) == 0


def test_table_lengths_validation(lib):
    # rh_rows / rw_rows: stored table lengths of the relative position (0 =
    # the needed 2*max-1); other kinds must leave them 0.
    bf = torch.bfloat16
    q = t(1, 2, 196, 64, dtype=bf)
    for nh, nw in [(27, 27), (15, 31), (1, 1), (127, 63)]:
        rb = B.RelposBias(t(nh, 64, dtype=bf), t(nw, 64, dtype=bf), (14, 14))
        assert B.check(q, q.clone(), q.clone(), bias=rb) == 0, (nh, nw)
    rb = B.RelposBias(t(27, 64, dtype=bf), t(27, 64, dtype=bf), (14, 14))
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(q, q.clone(), q.clone(), q.clone(), rb, None,
                                                  "batched", None)
    h = B.lib()
    args = lambda: (ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                    ctypes.byref(md), ctypes.byref(oc), dt)
    assert (bd.rh_rows, bd.rw_rows) == (27, 27)
    bd.rh_rows = 0
    assert h.attn_check(*args()) == 0      # 0: the needed length
    bd.rh_rows = -1
    assert h.attn_check(*args()) == 2
    bd.rh_rows = 1024
    assert h.attn_check(*args()) == 4
    bd.rh_rows = 27
    tab = t(27 * 27, 2, dtype=bf)
    bd.kind, bd.table = 1, tab.data_ptr()  # a table bias with table lengths set
    assert h.attn_check(*args()) == 2
    del keep


def test_backward_validation(lib):
    # attn_bwd_check: the gradients are shaped like q, k, v, must not
    # overlap inputs or each other; a table bias needs dtable and a
    # workspace of B_eff*H*rows*4 bytes; only window units in half
    # precision are built.
    h = B.lib()
    q, k, v, do = (t(4, 3, 49, 32) for _ in range(4))
    dq, dk, dv = t(4, 3, 49, 32), t(4, 3, 49, 32), t(4, 3, 49, 32)
    tab = B.TableBias(t(169, 3), (7, 7))
    dtab = torch.zeros(169, 3)
    ws = torch.zeros(4 * 3 * 169 * 4 // 4)  # float32 elements: exactly the bytes needed
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(q, k, v, do, tab, None, "batched", None)
    T = lambda x: B._tensor_c(x, 0)
    dqc, dkc, dvc = T(dq), T(dk), T(dv)
    def chk(dtable=dtab, w=ws, wbytes=None, dqx=None):
        return h.attn_bwd_check(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(oc),
                                ctypes.byref(bd), ctypes.byref(md), ctypes.byref(dqx or dqc),
                                ctypes.byref(dkc), ctypes.byref(dvc),
                                ctypes.c_void_p(dtable.data_ptr() if dtable is not None else 0), dt,
                                ctypes.c_void_p(w.data_ptr() if w is not None else 0),
                                ctypes.c_size_t(w.numel() * 4 if (w is not None and wbytes is None) else (wbytes or 0)))
    need = ctypes.c_size_t(0)
    assert h.attn_bwd_workspace_size(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(oc),
                                     ctypes.byref(bd), ctypes.byref(md), dt, ctypes.byref(need)) == 0
    assert need.value == 4 * 3 * 169 * 4
    assert chk() == 0
    assert chk(dtable=None) == 1                       # table gradient output missing
    assert chk(w=None) == 1                            # workspace missing
    assert chk(wbytes=need.value - 4) == 2             # workspace too small
    assert chk(dqx=T(q)) == 5                          # dq is q
    assert chk(dqx=T(t(4, 3, 50, 32))) == 2            # dq shaped unlike q
    ins = [t(1, 2, 100, 64) for _ in range(4)]  # kept alive: distinct addresses
    qc2, kc2, vc2, bd2, md2, oc2, dt2, keep2 = B._marshal(*ins, None, None, "batched", None)
    grads = [t(1, 2, 100, 64) for _ in range(3)]  # kept alive: distinct addresses
    d1, d2, d3 = (T(x) for x in grads)
    # Longer than a window without bias: the tiled backward, whose workspace
    # holds each row's log-sum-exp and D (2 * B * H * Nq floats).
    args2 = lambda w, n: (ctypes.byref(qc2), ctypes.byref(kc2), ctypes.byref(vc2), ctypes.byref(oc2),
                          ctypes.byref(bd2), ctypes.byref(md2), ctypes.byref(d1), ctypes.byref(d2),
                          ctypes.byref(d3), None, dt2, w, n)
    assert h.attn_bwd_check(*args2(None, 0)) == 1
    wsl = torch.zeros(2 * 1 * 2 * 100)
    assert h.attn_bwd_check(*args2(ctypes.c_void_p(wsl.data_ptr()), 2 * 2 * 100 * 4)) == 0
    # The relative position on a long sequence (10x10 grid, equal key grid,
    # tables of 19 rows): dtable = [dRh; dRw] (19 + 19 rows of d floats) and
    # a workspace of L, D (2*B*H*Nq), the rel_h / rel_w rows (B*H*Nq*32 when
    # gh + gw <= 32 and Nk <= 256, else B*H*Nq*(gh+gw)) and one partial per
    # 64 query rows (B*H*ceil(Nq/64)*(19+19)*d), each region rounded up to 4
    # floats.
    rb = B.RelposBias(t(19, 64), t(19, 64), (10, 10))
    qc3, kc3, vc3, bd3, md3, oc3, dt3, keep3 = B._marshal(*ins, rb, None, "batched", None)
    need3 = ctypes.c_size_t(0)
    assert h.attn_bwd_workspace_size(ctypes.byref(qc3), ctypes.byref(kc3), ctypes.byref(vc3),
                                     ctypes.byref(oc3), ctypes.byref(bd3), ctypes.byref(md3), dt3,
                                     ctypes.byref(need3)) == 0
    up4 = lambda n: (n + 3) // 4 * 4
    assert need3.value == 4 * (up4(up4(2 * 2 * 100) + 2 * 100 * 32) + 2 * 2 * 38 * 64)
    rb18 = B.RelposBias(t(35, 64), t(31, 64), (18, 16))     # gh + gw = 34: (gh + gw) floats a query
    q18 = t(1, 2, 18 * 16, 64)
    m18 = B._marshal(q18, q18.clone(), q18.clone(), q18.clone(), rb18, None, "batched", None)
    need18 = ctypes.c_size_t(0)
    assert h.attn_bwd_workspace_size(ctypes.byref(m18[0]), ctypes.byref(m18[1]), ctypes.byref(m18[2]),
                                     ctypes.byref(m18[5]), ctypes.byref(m18[3]), ctypes.byref(m18[4]), m18[6],
                                     ctypes.byref(need18)) == 0
    assert need18.value == 4 * (up4(up4(2 * 2 * 288) + 2 * 288 * 34) + 2 * 5 * 66 * 64)
    del m18
    dr = torch.zeros(38, 64)
    wsr = torch.zeros(need3.value // 4)
    args3 = lambda dtab, n: (ctypes.byref(qc3), ctypes.byref(kc3), ctypes.byref(vc3), ctypes.byref(oc3),
                             ctypes.byref(bd3), ctypes.byref(md3), ctypes.byref(d1), ctypes.byref(d2),
                             ctypes.byref(d3), dtab, dt3, ctypes.c_void_p(wsr.data_ptr()), n)
    assert h.attn_bwd_check(*args3(ctypes.c_void_p(dr.data_ptr()), need3.value)) == 0
    assert h.attn_bwd_check(*args3(None, need3.value)) == 1              # no [dRh; dRw] output
    assert h.attn_bwd_check(*args3(ctypes.c_void_p(dr.data_ptr()), need3.value - 4)) == 2
    # 64-wide grids: each partial slot holds at least (gh + 64) * 64 floats
    # (the workgroup's dRelH and dRelW before its partial).  A 4x64 grid at
    # d = 32: slots of max((7 + 127) * 32, 68 * 64) = 4352 floats.
    def ws_need(qq, bias):
        m = B._marshal(qq, qq.clone(), qq.clone(), qq.clone(), bias, None, "batched", None)
        n = ctypes.c_size_t(0)
        assert h.attn_bwd_workspace_size(ctypes.byref(m[0]), ctypes.byref(m[1]), ctypes.byref(m[2]),
                                         ctypes.byref(m[5]), ctypes.byref(m[3]), ctypes.byref(m[4]), m[6],
                                         ctypes.byref(n)) == 0
        return n.value
    q4 = t(2, 3, 4 * 64, 32)
    n4 = 2 * 3 * 4 * 64
    assert ws_need(q4, B.RelposBias(t(7, 32), t(127, 32), (4, 64))) == \
        4 * (up4(up4(2 * n4) + n4 * 68) + 2 * 3 * 4 * 4352)
    q8 = t(1, 2, 8 * 64, 64)       # d = 64: the [dRh; dRw] part is the larger
    n8 = 1 * 2 * 8 * 64
    assert ws_need(q8, B.RelposBias(t(15, 64), t(127, 64), (8, 64))) == \
        4 * (up4(up4(2 * n8) + n8 * 72) + 1 * 2 * 8 * (15 + 127) * 64)
    # Not built: keys on their own grid, resized tables, a mask, the image
    # layout beyond windows, and general grids with gh + gw > 84.
    def bwd_status(qq, kk, bias, mask=None, layout="batched", window=None):
        args = B._marshal(qq, kk, kk.clone(), qq.clone(), bias, mask, layout, window)
        qx, kx, vx, bx, mx, ox, dx, kp = args
        n = ctypes.c_size_t(0)
        return h.attn_bwd_workspace_size(ctypes.byref(qx), ctypes.byref(kx), ctypes.byref(vx), ctypes.byref(ox),
                                         ctypes.byref(bx), ctypes.byref(mx), dx, ctypes.byref(n))
    q100, k64 = t(1, 2, 100, 64), t(1, 2, 64, 64)
    assert bwd_status(q100, k64, B.RelposBias(t(19, 64), t(19, 64), (10, 10), (8, 8))) == 4
    assert bwd_status(q100, q100, B.RelposBias(t(27, 64), t(19, 64), (10, 10))) == 4
    assert bwd_status(q100, q100, rb, mask=B.AdditiveMask(t(1, 100, 100))) == 4
    q2500 = t(1, 1, 2500, 32)
    assert bwd_status(q2500, q2500, B.RelposBias(t(99, 32), t(99, 32), (50, 50))) == 4
    q1600 = t(1, 1, 1600, 32)
    assert bwd_status(q1600, q1600, B.RelposBias(t(79, 32), t(79, 32), (40, 40))) == 0   # gh + gw = 80
    q4096 = t(1, 1, 4096, 64)
    assert bwd_status(q4096, q4096, B.RelposBias(t(127, 64), t(127, 64), (64, 64))) == 0  # 64-wide form
    # The general form's LDS bound: gh + gw = 84 fits up to d = 64; at d = 80
    # the larger staged tiles leave room for 83.
    q42 = t(1, 1, 42 * 42, 64)
    assert bwd_status(q42, q42, B.RelposBias(t(83, 64), t(83, 64), (42, 42))) == 0
    q42 = t(1, 1, 42 * 42, 80)
    assert bwd_status(q42, q42, B.RelposBias(t(83, 80), t(83, 80), (42, 42))) == 4
    q4241 = t(1, 1, 42 * 41, 80)
    assert bwd_status(q4241, q4241, B.RelposBias(t(83, 80), t(81, 80), (42, 41))) == 0
    q43 = t(1, 1, 43 * 42, 32)
    assert bwd_status(q43, q43, B.RelposBias(t(85, 32), t(83, 32), (43, 42))) == 4
    # Small general grids (gh + gw <= 32, at most 256 keys) take the one-hot
    # key table's form: its largest case fits at d = 80 too.
    q256 = t(1, 1, 16 * 16, 80)
    assert bwd_status(q256, q256, B.RelposBias(t(31, 80), t(31, 80), (16, 16))) == 0
    qi = t(1, 2, 64 * 64, 64)
    img = B.Window(64, 64, 14, 14, 0, 0)
    assert bwd_status(qi, qi, B.RelposBias(t(27, 64), t(27, 64), (14, 14)), layout="image", window=img) == 4
    del keep, keep2, keep3


def test_e4m3_inputs_validation(lib):
    # q, k, v as 8-bit E4M3 codes with one scale each (options.qkv_format);
    # the compute and output dtype is the call's dtype (f16 or bf16).
    def q8(*shape):
        return torch.zeros(*shape, dtype=torch.uint8)
    sc = (0.01, 0.02, 0.03)
    geom = B.Window(56, 56, 7, 7, 3, 3)
    qi = q8(2, 3, 56 * 56, 32)
    tab = B.TableBias(t(169, 3), (7, 7))
    # The Swin-T shifted windows, image layout.
    assert B.check(qi, qi.clone(), qi.clone(), bias=tab, mask=B.ShiftMask(geom), layout="image",
                   qkv_descale=sc) == 0
    # SD self- and cross-attention, d = 40: rows of 40 bytes (8-byte aligned).
    qs = q8(2, 8, 4096, 40)
    assert B.check(qs, qs.clone(), qs.clone(), qkv_descale=sc) == 0
    kx = q8(2, 8, 77, 40)
    assert B.check(qs, kx, kx.clone(), qkv_descale=sc) == 0
    assert B.check(qs, kx, kx.clone(), qkv_descale=sc, out_dtype=torch.bfloat16) == 0
    # float8_e4m3fn tensors are taken as the same codes.
    qe = qs.view(torch.float8_e4m3fn)
    assert B.check(qe, qe.clone(), qe.clone(), qkv_descale=sc) == 0
    # Scales must be finite and positive.
    for bad in [(0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, float("nan")), (float("inf"), 1.0, 1.0)]:
        assert B.check(qs, qs.clone(), qs.clone(), qkv_descale=bad) == 7, bad
    # No fp32 compute, no relative position, no packed windows with 8-bit inputs.
    assert B.check(qs, qs.clone(), qs.clone(), qkv_descale=sc, out_dtype=torch.float32) == 4
    g = q8(1, 2, 196, 64)
    rel = B.RelposBias(t(27, 64), t(27, 64), (14, 14))
    assert B.check(g, g.clone(), g.clone(), bias=rel, qkv_descale=sc) == 4
    w = q8(4, 3, 49, 32)
    assert B.check(w, w.clone(), w.clone(), bias=tab, qkv_descale=sc) == 0
    assert B.check(w, w.clone(), w.clone(), bias=tab, qkv_descale=sc, window_heads=3) == 4
    # 8-byte alignment: a stride of 8 elements is fine, 4 is not; a base
    # pointer 8 bytes past a 16-byte boundary is fine, 4 bytes is not.
    buf = q8(2 * 8 * 77 * 48 + 16)
    k48 = buf[:2 * 8 * 77 * 48].view(2, 8, 77, 48)[..., :40]
    assert B.check(qs, k48, k48, qkv_descale=sc) == 0
    k44 = buf[:2 * 8 * 77 * 44].view(2, 8, 77, 44)[..., :40]
    assert B.check(qs, k44, k44, qkv_descale=sc) == 3
    base = q8(2 * 8 * 77 * 40 + 64)
    off = (-base.data_ptr()) % 16
    k_plus8 = base[off + 8:off + 8 + 2 * 8 * 77 * 40].view(2, 8, 77, 40)
    assert B.check(qs, k_plus8, k_plus8.clone(), qkv_descale=sc) == 0
    k_plus4 = base[off + 4:off + 4 + 2 * 8 * 77 * 40].view(2, 8, 77, 40)
    assert B.check(qs, k_plus4, kx, qkv_descale=sc) == 3
    # An unknown format is an invalid field; dtype tensors with a format of
    # codes (or codes without it) are refused by the binding.
    o = B.OptionsC()
    o.qkv_format = 2
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(qs, qs, qs, t(2, 8, 4096, 40), None, None, "batched",
                                                 None, True)
    assert lib.attn_check_opt(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                              ctypes.byref(md), ctypes.byref(oc), dt, ctypes.byref(o)) == 7
    with pytest.raises(TypeError):
        B.check(t(2, 8, 4096, 40), qs, qs, qkv_descale=sc)
    with pytest.raises(TypeError):
        B.check(qs, qs.clone(), qs.clone())
    # out may not overlap the codes: their extent is counted in bytes.
    raw = torch.zeros(2 * 8 * 4096 * 40 * 3, dtype=torch.uint8)
    qa = raw[:2 * 8 * 4096 * 40].view(2, 8, 4096, 40)
    oa = raw.view(torch.float16)[:2 * 8 * 4096 * 40].view(2, 8, 4096, 40)
    assert B.check(qa, qs, qs.clone(), out=oa, qkv_descale=sc) == 5
    ob = raw.view(torch.float16)[2 * 8 * 4096 * 40 // 2:].view(2, 8, 4096, 40)  # starts past q's bytes
    assert B.check(qa, qs, qs.clone(), out=ob, qkv_descale=sc) == 0


def test_lse_output_validation(lib):
    # The per-row log-sum-exp output: fp32 [B, H, N], 4-byte aligned, no
    # overlap; half precision and the one-head window form only.
    q = t(2, 3, 300, 64)
    lse = torch.zeros(2, 3, 300)
    assert B.check(q, q.clone(), q.clone(), lse=lse) == 0
    qw = t(4, 3, 49, 32)
    lw = torch.zeros(4, 3, 49)
    assert B.check(qw, qw.clone(), qw.clone(), lse=lw) == 0
    assert B.check(qw, qw.clone(), qw.clone(), lse=lw, window_heads=3) == 4
    qf = t(2, 3, 300, 64, dtype=torch.float32)
    assert B.check(qf, qf.clone(), qf.clone(), lse=lse) == 4
    # Image layout: [images, H, img_h*img_w].
    qi = t(2, 3, 56 * 56, 32)
    tab = B.TableBias(t(169, 3), (7, 7))
    geom = B.Window(56, 56, 7, 7, 3, 3)
    assert B.check(qi, qi.clone(), qi.clone(), bias=tab, mask=B.ShiftMask(geom), layout="image",
                   lse=torch.zeros(2, 3, 56 * 56)) == 0
    # Misaligned and overlapping outputs, through the C entry point.
    raw = torch.zeros(2 * 3 * 300 + 4)
    o = B.OptionsC()
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(q, q.clone(), q.clone(), t(2, 3, 300, 64), None, None,
                                                 "batched", None)
    def st(ptr):
        o.lse = ptr
        return lib.attn_check_opt(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                                  ctypes.byref(md), ctypes.byref(oc), dt, ctypes.byref(o))
    assert st(raw.data_ptr()) == 0
    assert st(raw.data_ptr() + 2) == 3
    assert st(q.data_ptr()) == 5          # over q
    del keep


def test_backward_options_validation(lib):
    # attn_bwd_opt: out and lse together (one alone: E_NULL), out shaped like
    # dout, lse 4-byte aligned, neither overlapping a gradient.  Only calls
    # that validation refuses are made here (they return before any HIP call).
    h = B.lib()
    ins = [t(1, 2, 300, 64) for _ in range(4)]
    grads = [t(1, 2, 300, 64) for _ in range(3)]
    fo, lse = t(1, 2, 300, 64), torch.zeros(1, 2, 300 + 4)
    qc, kc, vc, bd, md, oc, dt, keep = B._marshal(*ins, None, None, "batched", None)
    T = lambda x: B._tensor_c(x, 0)
    d1, d2, d3 = (T(x) for x in grads)
    ws = torch.zeros(2 * 2 * 300)

    def st(out_t, lse_ptr):
        bo = B.BwdOptionsC()
        foc = T(out_t) if out_t is not None else None
        bo.out = ctypes.addressof(foc) if foc is not None else None
        bo.lse = lse_ptr
        return h.attn_bwd_opt(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(oc),
                              ctypes.byref(bd), ctypes.byref(md), ctypes.byref(d1), ctypes.byref(d2),
                              ctypes.byref(d3), None, dt, ctypes.byref(bo), ctypes.c_void_p(ws.data_ptr()),
                              ws.numel() * 4, None)
    assert st(fo, None) == 1                          # lse missing
    assert st(None, lse.data_ptr()) == 1              # out missing
    assert st(t(1, 2, 299, 64), lse.data_ptr()) == 2  # out not shaped like dout
    assert st(fo, lse.data_ptr() + 2) == 3            # lse misaligned
    assert st(grads[0], lse.data_ptr()) == 5          # out is dq
    assert st(fo, grads[1].data_ptr()) == 5           # lse inside dk
    del keep
