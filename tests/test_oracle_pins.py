"""Pins for the fp64 oracle (CPU only).

The pages print no worked numeric example for attention, so the oracle is
pinned by routes that do not share its code: pure-Python scalar brute force on
tiny inputs (independent index derivations), closed forms, invariants of the
softmax, and a library routine (torch's CPU scaled_dot_product_attention in
float64) for the cases that reduce to it.  Each test names the mistake it
would catch.
"""

import math
import itertools

import numpy as np
import pytest
import torch

import oracle as O


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# Pure-Python brute force (no numpy in the arithmetic)
# ---------------------------------------------------------------------------

def py_softmax_combine(logits, vrows):
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    s = sum(e)
    d = len(vrows[0])
    return [sum(e[j] / s * vrows[j][c] for j in range(len(e))) for c in range(d)]


def py_dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def py_offsets_index(gh, gw):
    """Relative offset (dh, dw) -> table row, by enumerating all offsets in order."""
    offs = [(dh, dw) for dh in range(-(gh - 1), gh) for dw in range(-(gw - 1), gw)]
    return {o: i for i, o in enumerate(offs)}


def py_attention_window(q, k, v, gh, gw, table=None, h=0, rh=None, rw=None, labels=None,
                        value=-100.0):
    """One (batch item, head): q,k,v are lists of rows; tokens row-major on gh x gw."""
    d = len(q[0])
    scale = 1.0 / math.sqrt(d)
    idx = py_offsets_index(gh, gw)
    out = []
    for i in range(len(q)):
        qi_r, qi_c = divmod(i, gw)
        logits = []
        for j in range(len(k)):
            kj_r, kj_c = divmod(j, gw)
            s = scale * py_dot(q[i], k[j])
            if table is not None:
                s += table[idx[(qi_r - kj_r, qi_c - kj_c)]][h]
            if rh is not None:
                s += py_dot(q[i], rh[qi_r - kj_r + gh - 1]) + py_dot(q[i], rw[qi_c - kj_c + gw - 1])
            if labels is not None and labels[i] != labels[j]:
                s += value
            logits.append(s)
        out.append(py_softmax_combine(logits, v))
    return out


def tolist2(a):
    return [[float(x) for x in row] for row in a]


def test_bruteforce_plain_and_cross():
    # N=2 and 4 queries, cross-attention with 3 keys: catches a transposed QK^T
    # or a missing scale.
    for (nq, nk, d, seed) in [(2, 2, 3, 0), (4, 4, 5, 1), (4, 3, 2, 2)]:
        q, k, v = rnd((1, 1, nq, d), seed), rnd((1, 1, nk, d), seed + 10), rnd((1, 1, nk, 4), seed + 20)
        got = O.attention(q, k, v)[0, 0]
        d_ = d
        scale = 1 / math.sqrt(d_)
        exp = [py_softmax_combine([scale * py_dot(qi, kj) for kj in tolist2(k[0, 0])], tolist2(v[0, 0]))
               for qi in tolist2(q[0, 0])]
        np.testing.assert_allclose(got, np.array(exp), rtol=0, atol=1e-12)


@pytest.mark.parametrize("gh,gw", [(2, 2), (2, 3), (3, 2)])
def test_bruteforce_table_bias(gh, gw):
    # Catches a wrong offset sign, a swapped row/column or a wrong flattening
    # of the relative-position table (the brute force enumerates offsets).
    H, d, N = 2, 4, gh * gw
    q, k, v = rnd((1, H, N, d), 3), rnd((1, H, N, d), 4), rnd((1, H, N, d), 5)
    table = rnd(((2 * gh - 1) * (2 * gw - 1), H), 6)
    got = O.attention(q, k, v, bias=O.Bias("table", grid=(gh, gw), table=table))
    for h in range(H):
        exp = py_attention_window(tolist2(q[0, h]), tolist2(k[0, h]), tolist2(v[0, h]), gh, gw,
                                  table=tolist2(table), h=h)
        np.testing.assert_allclose(got[0, h], np.array(exp), rtol=0, atol=1e-12)


@pytest.mark.parametrize("gh,gw", [(2, 3), (3, 3)])
def test_bruteforce_relpos_bias(gh, gw):
    # Catches scaling q inside the bias, using key-query instead of
    # query-key, or swapping Rh and Rw.
    H, d, N = 2, 3, gh * gw
    q, k, v = rnd((2, H, N, d), 7), rnd((2, H, N, d), 8), rnd((2, H, N, d), 9)
    rh, rw = rnd((2 * gh - 1, d), 10), rnd((2 * gw - 1, d), 11)
    got = O.attention(q, k, v, bias=O.Bias("relpos", grid=(gh, gw), rh=rh, rw=rw))
    for b, h in itertools.product(range(2), range(H)):
        exp = py_attention_window(tolist2(q[b, h]), tolist2(k[b, h]), tolist2(v[b, h]), gh, gw,
                                  rh=tolist2(rh), rw=tolist2(rw))
        np.testing.assert_allclose(got[b, h], np.array(exp), rtol=0, atol=1e-12)


def test_bruteforce_image_shift_window():
    # 6x6 image, 3x3 windows, shift 1, table bias and region mask, checked
    # against a scalar implementation that follows pixels explicitly: window
    # (wy, wx), token (ty, tx) reads image pixel ((wy*3+ty+1) % 6,
    # (wx*3+tx+1) % 6) and labels come from per-pixel comparisons.  Catches a
    # wrong roll direction, a wrong region boundary or a wrong window order.
    ih = iw = 6
    wh = ww = 3
    sh = sw = 1
    B, H, d = 2, 2, 4
    q, k, v = (rnd((B, H, ih * iw, d), s) for s in (12, 13, 14))
    table = rnd(((2 * wh - 1) * (2 * ww - 1), H), 15)
    win = (ih, iw, wh, ww, sh, sw)
    got = O.attention_image(q, k, v, win, bias=O.Bias("table", grid=(wh, ww), table=table),
                            mask=O.Mask("shift", window=win))

    def region(y, x):
        ry = 0 if y < ih - wh else (1 if y < ih - sh else 2)
        rx = 0 if x < iw - ww else (1 if x < iw - sw else 2)
        return 3 * ry + rx

    exp = np.zeros_like(got)
    for b in range(B):
        for h in range(H):
            for wy in range(ih // wh):
                for wx in range(iw // ww):
                    pix, labels = [], []
                    for ty in range(wh):
                        for tx in range(ww):
                            y, x = wy * wh + ty, wx * ww + tx
                            pix.append(((y + sh) % ih) * iw + (x + sw) % iw)
                            labels.append(region(y, x))
                    qw = [[float(c) for c in q[b, h, p]] for p in pix]
                    kw = [[float(c) for c in k[b, h, p]] for p in pix]
                    vw = [[float(c) for c in v[b, h, p]] for p in pix]
                    ow = py_attention_window(qw, kw, vw, wh, ww, table=tolist2(table), h=h,
                                             labels=labels)
                    for t, p in enumerate(pix):
                        exp[b, h, p] = ow[t]
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-12)


def _py_padded_image(q, k, v, ih, iw, wh, ww, sh, sw, **kw):
    """Scalar reference for the padded image layout: the grid is padded to
    whole windows (ph, pw); window (wy, wx), token (ty, tx) reads padded pixel
    ((wy*wh+ty+sh) % ph, (wx*ww+tx+sw) % pw), a zero vector when that pixel is
    outside the image, and only real pixels receive an output."""
    ph, pw = -(-ih // wh) * wh, -(-iw // ww) * ww
    B, H, _, d = q.shape
    regions = kw.pop("regions", False)

    def region(y, x):
        ry = 0 if y < ph - wh else (1 if y < ph - sh else 2)
        rx = 0 if x < pw - ww else (1 if x < pw - sw else 2)
        return 3 * ry + rx

    exp = np.full(q.shape, np.nan)
    for b in range(B):
        for h in range(H):
            for wy in range(ph // wh):
                for wx in range(pw // ww):
                    pix, labels, qw, kwn, vw = [], [], [], [], []
                    for ty in range(wh):
                        for tx in range(ww):
                            y, x = wy * wh + ty, wx * ww + tx
                            py_, px_ = (y + sh) % ph, (x + sw) % pw
                            real = py_ < ih and px_ < iw
                            p_ = py_ * iw + px_ if real else None
                            pix.append(p_)
                            labels.append(region(y, x))
                            for dst, src in ((qw, q), (kwn, k), (vw, v)):
                                dst.append([float(c) for c in src[b, h, p_]] if real else [0.0] * d)
                    ow = py_attention_window(qw, kwn, vw, wh, ww, h=h,
                                             labels=labels if regions else None, **kw)
                    for t, p_ in enumerate(pix):
                        if p_ is not None:
                            exp[b, h, p_] = ow[t]
    return exp


def test_bruteforce_padded_image_shift_window():
    # 5x4 image, 3x3 windows -> padded 6x6, shift 1, table bias and region
    # mask (regions of the padded grid).  Catches padding on the wrong side,
    # a shift taken modulo the unpadded size, labels from the unpadded size,
    # or padding tokens masked out instead of attended as zero vectors.
    ih, iw, wh, ww, sh, sw = 5, 4, 3, 3, 1, 1
    B, H, d = 2, 2, 4
    q, k, v = (rnd((B, H, ih * iw, d), s) for s in (60, 61, 62))
    table = rnd(((2 * wh - 1) * (2 * ww - 1), H), 63)
    win = (ih, iw, wh, ww, sh, sw)
    got = O.attention_image(q, k, v, win, bias=O.Bias("table", grid=(wh, ww), table=table),
                            mask=O.Mask("shift", window=win))
    exp = _py_padded_image(q, k, v, ih, iw, wh, ww, sh, sw, table=tolist2(table), regions=True)
    assert not np.isnan(exp).any()
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-12)


def test_bruteforce_padded_image_relpos():
    # 4x5 image in 3x3 windows (padded 6x6), decomposed relative position,
    # no shift: padding queries are zero, so their own bias rows vanish, but
    # real queries still add q.Rh + q.Rw towards padding keys.
    ih, iw, wh, ww = 4, 5, 3, 3
    B, H, d = 1, 2, 4
    q, k, v = (rnd((B, H, ih * iw, d), s) for s in (64, 65, 66))
    rh, rw = rnd((2 * wh - 1, d), 67), rnd((2 * ww - 1, d), 68)
    win = (ih, iw, wh, ww, 0, 0)
    got = O.attention_image(q, k, v, win, bias=O.Bias("relpos", grid=(wh, ww), rh=rh, rw=rw))
    exp = _py_padded_image(q, k, v, ih, iw, wh, ww, 0, 0, rh=tolist2(rh), rw=tolist2(rw))
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-12)


def test_padding_keys_add_to_the_denominator_only():
    # Closed form: without a bias a padding key has logit 0 and value 0, so a
    # window with n_pad padding tokens gives, for a real query,
    #   o = sum_real e^{s_j} v_j / (sum_real e^{s_j} + n_pad).
    # 2x3 image in 2x2 windows -> padded 2x4: the second window holds pixels
    # (0,2), (1,2) and two padding tokens.
    ih, iw = 2, 3
    d = 3
    q, k, v = (rnd((1, 1, ih * iw, d), s) for s in (69, 70, 71))
    got = O.attention_image(q, k, v, (ih, iw, 2, 2, 0, 0))
    real = [2, 5]  # image pixels of the second window
    scale = 1 / math.sqrt(d)
    for i in real:
        s = np.array([scale * q[0, 0, i] @ k[0, 0, j] for j in real])
        e = np.exp(s)
        exp = (e[:, None] * v[0, 0, real]).sum(0) / (e.sum() + 2.0)
        np.testing.assert_allclose(got[0, 0, i], exp, rtol=0, atol=1e-13)


def test_bruteforce_additive_bias_and_mask():
    B, H, nq, nk, d = 3, 2, 3, 4, 2
    q, k, v = rnd((B, H, nq, d), 16), rnd((B, H, nk, d), 17), rnd((B, H, nk, d), 18)
    add_b = rnd((1, nq, nk), 19)
    add_m = rnd((3, nq, nk), 20)
    got = O.attention(q, k, v, bias=O.Bias("additive", add=add_b), mask=O.Mask("additive", add=add_m))
    scale = 1 / math.sqrt(d)
    for b, h in itertools.product(range(B), range(H)):
        for i in range(nq):
            logits = [scale * py_dot(q[b, h, i], k[b, h, j]) + add_b[0, i, j] + add_m[b % 3, i, j]
                      for j in range(nk)]
            exp = py_softmax_combine(logits, tolist2(v[b, h]))
            np.testing.assert_allclose(got[b, h, i], exp, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms and special cases
# ---------------------------------------------------------------------------

def test_two_token_closed_form():
    # o = sigmoid(s1 - s2) v1 + (1 - sigmoid) v2 (a dropped max-subtraction or
    # a wrong normaliser fails this).
    q, k, v = rnd((1, 1, 1, 8), 21), rnd((1, 1, 2, 8), 22), rnd((1, 1, 2, 5), 23)
    s = (q[0, 0, 0] @ k[0, 0].T) / math.sqrt(8)
    sig = 1 / (1 + math.exp(-(s[0] - s[1])))
    exp = sig * v[0, 0, 0] + (1 - sig) * v[0, 0, 1]
    np.testing.assert_allclose(O.attention(q, k, v)[0, 0, 0], exp, rtol=0, atol=1e-14)


def test_q_zero_gives_mean_of_v():
    # Q = 0: no bias -> mean of V; relpos bias is proportional to q -> still
    # the mean; table bias -> softmax(table row) . V.
    N, d = 9, 4
    q = np.zeros((1, 2, N, d))
    k, v = rnd((1, 2, N, d), 24), rnd((1, 2, N, d), 25)
    np.testing.assert_allclose(O.attention(q, k, v)[0], np.broadcast_to(v[0].mean(1, keepdims=True), (2, N, d)),
                               atol=1e-14)
    rb = O.Bias("relpos", grid=(3, 3), rh=rnd((5, d), 26), rw=rnd((5, d), 27))
    np.testing.assert_allclose(O.attention(q, k, v, bias=rb)[0],
                               np.broadcast_to(v[0].mean(1, keepdims=True), (2, N, d)), atol=1e-14)
    table = rnd((25, 2), 28)
    got = O.attention(q, k, v, bias=O.Bias("table", grid=(3, 3), table=table))
    for h in range(2):
        for i in range(N):
            ri, ci = divmod(i, 3)
            w = np.array([math.exp(table[(ri - j // 3 + 2) * 5 + (ci - j % 3 + 2), h]) for j in range(N)])
            np.testing.assert_allclose(got[0, h, i], (w / w.sum()) @ v[0, h], atol=1e-14)


def test_dominant_logit_selects_row():
    N, d = 16, 8
    q, k, v = rnd((1, 1, N, d), 29), rnd((1, 1, N, d), 30), rnd((1, 1, N, d), 31)
    add = np.zeros((1, N, N))
    jstar = (np.arange(N) * 5) % N
    add[0, np.arange(N), jstar] = 60.0 + 40.0   # far above every other logit
    got = O.attention(q, k, v, bias=O.Bias("additive", add=add))[0, 0]
    np.testing.assert_allclose(got, v[0, 0, jstar], atol=N * math.exp(-60))


def test_single_key_returns_v0():
    q, k, v = rnd((2, 3, 7, 5), 32), rnd((2, 3, 1, 5), 33), rnd((2, 3, 1, 5), 34)
    np.testing.assert_array_equal(O.attention(q, k, v), np.broadcast_to(v, (2, 3, 7, 5)))


def test_rows_sum_to_one():
    q, k = rnd((2, 2, 10, 4), 35), rnd((2, 2, 13, 4), 36)
    p = O.attention_probs(q, k, mask=O.Mask("additive", add=rnd((2, 10, 13), 37)))
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=13 * 1e-15)


def test_key_value_permutation_invariance_and_query_equivariance():
    q, k, v = rnd((1, 2, 6, 4), 38), rnd((1, 2, 9, 4), 39), rnd((1, 2, 9, 3), 40)
    add = rnd((1, 6, 9), 41)
    perm = np.random.default_rng(42).permutation(9)
    base = O.attention(q, k, v, bias=O.Bias("additive", add=add))
    permd = O.attention(q, k[:, :, perm], v[:, :, perm], bias=O.Bias("additive", add=add[:, :, perm]))
    np.testing.assert_allclose(base, permd, atol=1e-13)
    qp = np.random.default_rng(43).permutation(6)
    qperm = O.attention(q[:, :, qp], k, v, bias=O.Bias("additive", add=add[:, qp]))
    np.testing.assert_allclose(base[:, :, qp], qperm, atol=1e-13)


def test_bias_row_constant_shift_invariance():
    # table + c and Rh + u (same vector added to every row) add a per-query
    # constant to every logit of the row: the output must not change.
    N, d = 9, 4
    q, k, v = rnd((1, 2, N, d), 44), rnd((1, 2, N, d), 45), rnd((1, 2, N, d), 46)
    table = rnd((25, 2), 47)
    a = O.attention(q, k, v, bias=O.Bias("table", grid=(3, 3), table=table))
    b = O.attention(q, k, v, bias=O.Bias("table", grid=(3, 3), table=table + 3.7))
    np.testing.assert_allclose(a, b, atol=1e-13)
    rh, rw = rnd((5, d), 48), rnd((5, d), 49)
    u = rnd((d,), 50)
    a = O.attention(q, k, v, bias=O.Bias("relpos", grid=(3, 3), rh=rh, rw=rw))
    b = O.attention(q, k, v, bias=O.Bias("relpos", grid=(3, 3), rh=rh + u, rw=rw))
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_relpos_decomposed_equals_literal_gather():
    for (gh, gw, d) in [(3, 4, 5), (14, 14, 8)]:
        N = gh * gw
        q = rnd((N, d), 51)
        rh, rw = rnd((2 * gh - 1, d), 52), rnd((2 * gw - 1, d), 53)
        rows = np.arange(N)
        np.testing.assert_allclose(O.relpos_bias(q, rows, rh, rw, gh, gw),
                                   O.relpos_bias_gather(q, rows, rh, rw, gh, gw), atol=1e-12)


def test_relpos_one_hot_tables_reveal_offsets():
    # With q = e0 and Rh[r] = r * e0, Rw = 0, the bias equals the table row
    # used: (query row - key row) + gh - 1.
    gh, gw, d = 4, 5, 3
    N = gh * gw
    q = np.zeros((N, d))
    q[:, 0] = 1.0
    rh = np.zeros((2 * gh - 1, d))
    rh[:, 0] = np.arange(2 * gh - 1)
    rw = np.zeros((2 * gw - 1, d))
    b = O.relpos_bias(q, np.arange(N), rh, rw, gh, gw)
    for i in range(N):
        for j in range(N):
            assert b[i, j] == (i // gw) - (j // gw) + gh - 1


def test_shift_mask_equals_per_region_attention():
    # Masked window attention = ordinary attention inside each region (to e^-100).
    win = (14, 14, 7, 7, 3, 3)
    mask = O.Mask("shift", window=win)
    nW = 4
    q, k, v = rnd((nW, 1, 49, 6), 54), rnd((nW, 1, 49, 6), 55), rnd((nW, 1, 49, 6), 56)
    got = O.attention(q, k, v, mask=mask)
    lab = O.window_partition(O.shift_region_labels(*win)[None, None, :, :, None].astype(float), 7, 7)[:, 0, :, 0]
    for w in range(nW):
        for i in range(49):
            same = np.nonzero(lab[w] == lab[w, i])[0]
            s = q[w, 0, i] @ k[w, 0, same].T / math.sqrt(6)
            p = np.exp(s - s.max())
            np.testing.assert_allclose(got[w, 0, i], (p / p.sum()) @ v[w, 0, same], atol=1e-30 + 49 * math.exp(-90))


def test_table_index_structure():
    # 7x7: the zero offset sits at row 84 on the diagonal, opposite offsets sum
    # to 168, and all 169 rows are used.
    idx = O.table_relative_index(7, 7)
    assert np.all(np.diag(idx) == 6 * 13 + 6)
    assert np.all(idx + idx.T == 168)
    assert idx.min() == 0 and idx.max() == 168 and len(np.unique(idx)) == 169
    # (dh, dw) = (1, 0): query one row below the key -> row 84 + 13.
    assert idx[7, 0] == 84 + 13 and idx[1, 0] == 84 + 1


def test_swin_t_stage1_shift_mask_statistics():
    # 56x56 image, 7x7 windows, shift 3: 15 of 64 windows straddle a region
    # boundary; 11.87% of query/key pairs are masked; every query keeps at
    # least 9 unmasked keys (its own region).
    m = O.shift_mask(56, 56, 7, 7, 3, 3)
    affected = np.count_nonzero(np.any(m != 0, axis=(1, 2)))
    assert affected == 15
    frac = np.count_nonzero(m) / m.size
    assert abs(frac - 0.1187) < 5e-4
    assert (m == 0).sum(-1).min() == 9
    assert set(np.unique(m)) == {0.0, -100.0}


def test_image_layout_without_shift_is_plain_partition():
    # shift 0 and no mask: image attention equals windows-as-batch attention on
    # the partitioned tensor.
    B, H, d = 1, 2, 3
    q, k, v = (rnd((B, H, 36, d), s) for s in (57, 58, 59))
    table = rnd((25, H), 60)
    bias = O.Bias("table", grid=(3, 3), table=table)
    got = O.attention_image(q, k, v, (6, 6, 3, 3, 0, 0), bias=bias)
    part = lambda x: O.window_partition(x.reshape(B, H, 6, 6, d), 3, 3)
    ref = O.window_reverse(O.attention(part(q), part(k), part(v), bias=bias), 6, 6, 3, 3).reshape(B, H, 36, d)
    np.testing.assert_allclose(got, ref, atol=1e-14)


def test_matches_torch_sdpa_float64_library_routine():
    # With a dense additive term, the oracle reduces to torch's CPU
    # scaled_dot_product_attention (float mask added after scaling).
    q, k, v = rnd((2, 3, 11, 8), 61), rnd((2, 3, 17, 8), 62), rnd((2, 3, 17, 6), 63)
    add = rnd((2, 11, 17), 64)
    got = O.attention(q, k, v, bias=O.Bias("additive", add=add))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(add)[:, None])
    np.testing.assert_allclose(got, ref.numpy(), atol=1e-13)


def test_select_rows_matches_full():
    q, k, v = rnd((2, 2, 40, 4), 65), rnd((2, 2, 40, 4), 66), rnd((2, 2, 40, 4), 67)
    rb = O.Bias("relpos", grid=(5, 8), rh=rnd((9, 4), 68), rw=rnd((15, 4), 69))
    full = O.attention(q, k, v, bias=rb, row_block=7)
    sel = O.attention(q, k, v, bias=rb, select=[(1, 0, [3, 39, 0]), (0, 1, np.arange(5, 12))])
    np.testing.assert_allclose(sel[0], full[1, 0, [3, 39, 0]], atol=1e-14)
    np.testing.assert_allclose(sel[1], full[0, 1, 5:12], atol=1e-14)


# ---------------------------------------------------------------------------
# Relative position with query and key grids of different sizes (the
# coordinate scalers of the SAM write-ups)
# ---------------------------------------------------------------------------

def py_scaled_row(qc, kc, qn, kn):
    """Table row on axes of qn query and kn key positions where one count is
    a whole multiple of the other: the shorter axis's coordinates are
    multiplied by the ratio, the difference is shifted to start at 0."""
    if qn >= kn:
        assert qn % kn == 0
        r = qn // kn
        return qc - r * kc + r * (kn - 1)
    assert kn % qn == 0
    r = kn // qn
    return r * qc - kc + (kn - 1)


@pytest.mark.parametrize("qn,kn", [(1, 1), (5, 5), (7, 14), (14, 7), (2, 8), (9, 3), (64, 32)])
def test_scaled_rows_whole_ratios_closed_form(qn, kn):
    # Catches stretching the wrong axis, a missing shift, or a shift by the
    # query range instead of the scaled key range.
    rows = O.relpos_rows(qn, kn)
    for qc in range(qn):
        for kc in range(kn):
            assert rows[qc, kc] == py_scaled_row(qc, kc, qn, kn), (qc, kc)


@pytest.mark.parametrize("qn,kn", [(3, 2), (2, 3), (10, 4), (4, 10), (14, 9), (9, 14), (6, 6), (1, 5), (5, 1)])
def test_scaled_rows_properties(qn, kn):
    # Any grid sizes: rows rise with the query coordinate, fall with the key
    # coordinate, stay inside the 2*max-1 table, start at row 0 (first query,
    # last key), and a query step moves by at most max(kn/qn, 1) rounded up.
    rows = O.relpos_rows(qn, kn)
    n = 2 * max(qn, kn) - 1
    assert rows.min() == 0 and rows[0, kn - 1] == 0 and rows.max() <= n - 1
    assert (np.diff(rows, axis=0) >= 0).all() and (np.diff(rows, axis=1) <= 0).all()
    assert (np.diff(rows, axis=0) <= math.ceil(max(kn / qn, 1))).all()
    assert (np.diff(rows, axis=1) >= -math.ceil(max(qn / kn, 1))).all()
    # The last query and the first key use the largest row, which is the
    # scaled extents added: (qn-1)*max(kn/qn,1) + (kn-1)*max(qn/kn,1), floored.
    top = (qn - 1) * max(kn / qn, 1) + (kn - 1) * max(qn / kn, 1)
    assert rows[qn - 1, 0] == rows.max() == math.floor(top + 1e-9)


@pytest.mark.parametrize("qgrid,kgrid", [((2, 2), (4, 2)), ((4, 3), (2, 3)), ((2, 3), (3, 2))])
def test_bruteforce_relpos_unequal_grids(qgrid, kgrid):
    # Pure-Python attention over explicit pairs; whole ratios use the closed
    # form of py_scaled_row, the (2,3)/(3,2) case the floor written out.
    (gh, gw), (kgh, kgw) = qgrid, kgrid
    H, d = 2, 3
    Nq, Nk = gh * gw, kgh * kgw
    q, k, v = rnd((1, H, Nq, d), 21), rnd((1, H, Nk, d), 22), rnd((1, H, Nk, d), 23)
    rh, rw = rnd((2 * max(gh, kgh) - 1, d), 24), rnd((2 * max(gw, kgw) - 1, d), 25)
    got = O.attention(q, k, v, bias=O.Bias("relpos", grid=qgrid, kgrid=kgrid, rh=rh, rw=rw))

    def row(qc, kc, qn, kn):
        if qn % kn == 0 or kn % qn == 0:
            return py_scaled_row(qc, kc, qn, kn)
        # 2 query and 3 key positions: queries count 3/2 units each;
        # 3 query and 2 key positions: keys count 3/2 units each.
        if (qn, kn) == (2, 3):
            return math.floor(qc * 1.5 - kc + 2)
        assert (qn, kn) == (3, 2)
        return math.floor(qc - kc * 1.5 + 1.5)

    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        qq, kk, vv = tolist2(q[0, h]), tolist2(k[0, h]), tolist2(v[0, h])
        for i in range(Nq):
            qr, qcol = divmod(i, gw)
            logits = []
            for j in range(Nk):
                kr, kcol = divmod(j, kgw)
                s = scale * py_dot(qq[i], kk[j])
                s += py_dot(qq[i], rh[row(qr, kr, gh, kgh)]) + py_dot(qq[i], rw[row(qcol, kcol, gw, kgw)])
                logits.append(s)
            np.testing.assert_allclose(got[0, h, i], py_softmax_combine(logits, vv), rtol=0, atol=1e-12)


def test_unequal_grids_reduce_to_equal_grids():
    # kgrid equal to grid is the plain decomposed bias.
    q = rnd((6, 4), 30)
    rh, rw = rnd((5, 4), 31), rnd((3, 4), 32)
    a = O.relpos_bias(q, np.arange(6), rh, rw, 3, 2)
    b = O.relpos_bias(q, np.arange(6), rh, rw, 3, 2, 3, 2)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# Resizing a relative-position table to the length the grids need
# (rel_pos_resized of the SAM write-ups; reading: linear interpolation along
# the offset axis, end rows aligned)
# ---------------------------------------------------------------------------

def py_resize(rows, m):
    """Pure-Python resize: new row r at old position r*(L-1)/(m-1), split
    into its integer and fractional parts by exact integer division."""
    L = len(rows)
    out = []
    for r in range(m):
        if L == 1 or m == 1:
            out.append(list(rows[0]))
            continue
        num, den = r * (L - 1), m - 1
        i, rem = divmod(num, den)
        if i >= L - 1:
            out.append(list(rows[L - 1]))
            continue
        f = rem / den
        out.append([(1 - f) * a + f * b for a, b in zip(rows[i], rows[i + 1])])
    return out


@pytest.mark.parametrize("L,m", [(5, 5), (3, 7), (7, 3), (27, 15), (15, 27), (63, 127), (127, 63),
                                 (2, 9), (1, 5), (6, 1), (31, 27)])
def test_resize_bruteforce(L, m):
    # Catches an off-by-one in the position (m or L instead of m-1, L-1), a
    # swapped interpolation weight, or a floor in the wrong place.
    t = rnd((L, 3), L * 100 + m)
    got = O.rel_pos_resized(t, m)
    np.testing.assert_allclose(got, np.array(py_resize(tolist2(t), m)), rtol=0, atol=1e-13)


@pytest.mark.parametrize("L,m", [(4, 4), (3, 11), (11, 3), (127, 27), (27, 127)])
def test_resize_closed_forms(L, m):
    # Identity at equal length; affine tables a + b*i stay affine with the
    # same end rows, a + b*r*(L-1)/(m-1); constant tables stay constant.
    t = rnd((L, 4), 7)
    if L == m:
        np.testing.assert_array_equal(O.rel_pos_resized(t, m), t)
    a, b = rnd(4, 8), rnd(4, 9)
    aff = a[None, :] + b[None, :] * np.arange(L)[:, None]
    want = a[None, :] + b[None, :] * (np.arange(m) * (L - 1) / (m - 1))[:, None]
    np.testing.assert_allclose(O.rel_pos_resized(aff, m), want, rtol=0, atol=1e-12)
    got = O.rel_pos_resized(aff, m)
    np.testing.assert_allclose(got[0], aff[0], atol=1e-14)
    np.testing.assert_allclose(got[-1], aff[-1], atol=1e-12)
    np.testing.assert_allclose(O.rel_pos_resized(np.ones((L, 2)) * 3.5, m), 3.5, atol=1e-14)


@pytest.mark.parametrize("L,m", [(3, 7), (27, 15), (15, 27), (63, 127)])
def test_resize_matches_library_interpolation(L, m):
    # The reading equals torch's linear interpolation with aligned corners
    # (a library routine with the same definition), in float64.
    t = rnd((L, 5), 3)
    lib = torch.nn.functional.interpolate(torch.from_numpy(t).T[None], size=m, mode="linear",
                                          align_corners=True)[0].T.numpy()
    np.testing.assert_allclose(O.rel_pos_resized(t, m), lib, rtol=0, atol=1e-12)


def test_relpos_bias_resizes_tables():
    # A table of another length is resized to 2*max-1 rows before use: the
    # bias equals the bias of the explicitly resized table, and the
    # attention equals a pure-Python brute force over the resized rows.
    gh, gw, d = 3, 4, 3
    q = rnd((1, 2, gh * gw, d), 40)
    k, v = rnd((1, 2, gh * gw, d), 41), rnd((1, 2, gh * gw, d), 42)
    rh, rw = rnd((9, d), 43), rnd((3, d), 44)          # need 5 and 7 rows
    a = O.relpos_bias(q[0, 0], np.arange(gh * gw), rh, rw, gh, gw)
    b = O.relpos_bias(q[0, 0], np.arange(gh * gw), O.rel_pos_resized(rh, 5), O.rel_pos_resized(rw, 7),
                      gh, gw)
    np.testing.assert_array_equal(a, b)
    got = O.attention(q, k, v, bias=O.Bias("relpos", grid=(gh, gw), rh=rh, rw=rw))
    rh5, rw7 = py_resize(tolist2(rh), 5), py_resize(tolist2(rw), 7)
    for h in range(2):
        want = py_attention_window(tolist2(q[0, h]), tolist2(k[0, h]), tolist2(v[0, h]), gh, gw,
                                   rh=rh5, rw=rw7)
        np.testing.assert_allclose(got[0, h], want, rtol=0, atol=1e-12)


def test_logsumexp_matches_torch_and_normalises_the_probabilities():
    # L_i against torch.logsumexp of the same logits (a library routine), on
    # a table bias with a shift-free additive mask; and exp(s - L) are the
    # oracle's own softmax rows.
    r = np.random.default_rng(7)
    q, k = r.standard_normal((2, 3, 9, 4)), r.standard_normal((2, 3, 9, 4))
    table = r.standard_normal((25, 3))
    bias = O.Bias("table", grid=(3, 3), table=table)
    madd = r.standard_normal((2, 9, 9))
    mask = O.Mask("additive", add=madd)
    lse = O.attention_logsumexp(q, k, bias, mask)
    tb = O.table_bias(table, 3, 3)                          # [H, N, N]
    s = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) / 2.0
    s = s + torch.from_numpy(tb)[None] + torch.from_numpy(madd)[:, None]
    assert np.allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)
    p = O.attention_probs(q, k, bias, mask)
    assert np.allclose(np.exp(s.numpy() - lse[..., None]), p, rtol=0, atol=1e-12)


def test_logsumexp_closed_forms():
    # Q = 0: every logit is 0, L = log Nk; one key: L = scale * q.k.
    q = np.zeros((1, 1, 3, 8))
    k = np.random.default_rng(1).standard_normal((1, 1, 5, 8))
    assert np.allclose(O.attention_logsumexp(q, k), np.log(5.0))
    q1 = np.random.default_rng(2).standard_normal((1, 2, 4, 8))
    k1 = np.random.default_rng(3).standard_normal((1, 2, 1, 8))
    expect = np.einsum("bhqc,bhkc->bhq", q1, k1) / np.sqrt(8.0)
    assert np.allclose(O.attention_logsumexp(q1, k1), expect, rtol=0, atol=1e-12)


def test_image_logsumexp_follows_the_pixels():
    # 5x4 image in 3x3 windows (padded to 6x6), shift 1, table bias and
    # regions: every real pixel's L equals the log-sum-exp of its own row of
    # logits, found by brute force from the pixel's window (same scalar
    # brute force as the attention pin above).
    r = np.random.default_rng(11)
    window = (5, 4, 3, 3, 1, 1)
    q, k = r.standard_normal((1, 2, 20, 4)), r.standard_normal((1, 2, 20, 4))
    bias = O.Bias("table", grid=(3, 3), table=r.standard_normal((25, 2)))
    mask = O.Mask("shift", window=window)
    lse = O.attention_image_logsumexp(q, k, window, bias, mask)
    ph = pw = 6
    lab = O.shift_region_labels(ph, pw, 3, 3, 1, 1)
    for h in range(2):
        for pix in range(20):
            y, x = divmod(pix, 4)
            # shifted position of this pixel and its window
            sy, sx = (y - 1) % ph, (x - 1) % pw
            wy, wx = sy // 3, sx // 3
            logits = []
            for ty in range(3):
                for tx in range(3):
                    ky, kx = (wy * 3 + ty + 1) % ph, (wx * 3 + tx + 1) % pw
                    kvec = k[0, h, ky * 4 + kx] if ky < 5 and kx < 4 else np.zeros(4)
                    qvec = q[0, h, pix]
                    dh, dw = (sy % 3) - ty, (sx % 3) - tx
                    b = bias.table[(dh + 2) * 5 + (dw + 2), h]
                    same = lab[sy, sx] == lab[wy * 3 + ty, wx * 3 + tx]
                    logits.append(qvec @ kvec / 2.0 + b + (0.0 if same else -100.0))
            logits = np.array(logits)
            m = logits.max()
            assert abs(lse[0, h, pix] - (m + np.log(np.exp(logits - m).sum()))) < 1e-12
