"""Plain fp64 CPU oracle for fused scaled-dot-product attention with the
additive bias and mask used by vision transformers.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

What is computed, and the passage each step follows (page title, section):

* Attention itself -- queries and keys, through a softmax, give the attention
  map, whose values weight the value tensor; heads are independent copies
  ["Training and inference acceleration for large vision models" (Swin
  Transformer talk), section 1 "Swin Transformer introduction"].  The scaled
  form is the ``scaled_dot_product_attention`` function of
  ["Accelerated Diffusers with PyTorch 2.0", section "Accelerating
  transformer blocks"]; its default scale 1/sqrt(d) is used throughout.
  Bias and mask are added to the scaled logits, before the softmax.
* Self- and cross-attention: same computation, key/value length may differ
  from the query length [Swin talk, section 1].
* Window attention, the window shift and the relative-position bias table
  [Swin talk, section 1; the window partition/shift/merge operations are pure
  index mappings, section 2 "Swin Transformer training optimisation"].
* Decomposed relative position (SAM): per-query coordinates index the
  relative-position tables [“Accelerating Generative AI with PyTorch:
  Segment Anything, Fast”, section "Bfloat16 half precision (plus GPU syncs
  and batching)"]; the bias is q·Rh[qh-kh+gh-1] + q·Rw[qw-kw+gw-1].

Readings taken where the pages are silent (all are listed with reasons in the
design notes of the repository):

* token t of a gh x gw grid sits at row t // gw, column t % gw;
* windows are numbered row-major inside an image and images are outermost
  (batch item = image * n_windows + window);
* table row for offset (dh, dw) = query - key is (dh+gh-1)*(2gw-1) + (dw+gw-1),
  the table is [(2gh-1)(2gw-1), H] (column = head);
* the relative-position tables Rh [2gh-1, d], Rw [2gw-1, d] are shared by all
  heads and are dotted with the raw (unscaled) query;
* queries and keys on grids of different sizes (the coordinate scalers
  q_coords and k_coords that the SAM write-ups name, same section): the
  shorter axis is stretched onto the longer one and the table row is the
  floor of the scaled coordinate difference, in exact arithmetic
  (``relpos_rows``); the tables then hold 2*max(q, k)-1 rows per axis.  The
  write-ups also name a resize of the tables (rel_pos_resized) without giving
  its rule: a table of another length is resized to 2*max(q, k)-1 rows by
  linear interpolation along the offset axis with both end rows kept
  (``rel_pos_resized``);
* the shifted window attention rolls the image content by (-sh, -sw) before
  partitioning (shifted[y] = x[(y + sh) mod img_h]) and rolls back after;
  the region of a shifted-image pixel is 3*ry + rx, where ry is 0, 1, 2 for
  rows in [0, img_h-win_h), [img_h-win_h, img_h-sh), [img_h-sh, img_h) (same
  for columns); query/key pairs from different regions get an additive
  ``value`` (default -100);
* an image that is not a whole number of windows is zero-padded at the bottom
  and right up to whole windows before the shift and the partition (SAM's
  64x64 token grid in 14x14 windows becomes 70x70; the pages pad SAM's
  encoder input with zeros for static shapes, "Segment Anything, Fast",
  section "Torch.compile"): padding tokens have q = k = v = 0, take part in
  the attention like any other token, and their outputs are cropped away;
  the shift and the region labels are taken on the padded grid;
* an additive bias of shape [nB, Nq, Nk] applies to batch item b as b % nB,
  an additive mask [nW, Nq, Nk] as b % nW;
* low-precision inputs: the SAM write-ups speed the model up with GPU
  quantization ("Segment Anything, Fast", introduction), and the Swin talk
  (section 3, inference optimisation) runs 8-bit matrix products whose
  quantization and dequantization are fused into the neighbouring
  operators.  Reading for this attention: q, k and v may arrive as 8-bit
  floating-point codes (E4M3 of the OCP 8-bit floating point
  specification), each tensor with one scale; the attention is computed on
  the dequantized values code * scale, exactly as on any other input, and
  the output has the compute dtype (``e4m3_decode``, ``dequantize_e4m3``).

Everything is numpy float64.  The inputs are the exact values the device
receives (already rounded to the device dtype), upcast to float64.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction
from typing import Optional, Sequence

import numpy as np


@dataclass
class Bias:
    """Additive bias description (mirrors the bias kinds of the attention call).

    kind: "none" | "table" | "relpos" | "additive"
    grid: (gh, gw) token grid of one batch item (table, relpos); for relpos
          the grid of the queries
    kgrid: relpos only, (kgh, kgw) grid of the keys; None means ``grid``
    table: [(2gh-1)(2gw-1), H]
    rh, rw: [2max(gh,kgh)-1, d], [2max(gw,kgw)-1, d]
    add: [nB, Nq, Nk], batch item b uses add[b % nB]
    """

    kind: str = "none"
    grid: Optional[tuple] = None
    kgrid: Optional[tuple] = None
    table: Optional[np.ndarray] = None
    rh: Optional[np.ndarray] = None
    rw: Optional[np.ndarray] = None
    add: Optional[np.ndarray] = None


@dataclass
class Mask:
    """Additive mask description.

    kind: "none" | "additive" | "shift"
    add: [nW, Nq, Nk], batch item b uses add[b % nW]
    window: (img_h, img_w, win_h, win_w, shift_h, shift_w)
    value: added to pairs from different shifted regions
    """

    kind: str = "none"
    add: Optional[np.ndarray] = None
    window: Optional[tuple] = None
    value: float = -100.0


# ---------------------------------------------------------------------------
# Index structure of windows and grids
# ---------------------------------------------------------------------------

def token_coords(gh: int, gw: int):
    """(row, col) of every token of a gh x gw grid, tokens in row-major order."""
    t = np.arange(gh * gw)
    return t // gw, t % gw


def table_relative_index(gh: int, gw: int) -> np.ndarray:
    """[N, N] row of the relative-position table used by query i and key j.

    Swin talk, section 1 (relative position bias); the offset is query minus
    key, shifted to be non-negative and flattened row-major over the
    (2gh-1) x (2gw-1) offsets.
    """
    r, c = token_coords(gh, gw)
    dh = r[:, None] - r[None, :]
    dw = c[:, None] - c[None, :]
    return (dh + gh - 1) * (2 * gw - 1) + (dw + gw - 1)


def table_bias(table: np.ndarray, gh: int, gw: int) -> np.ndarray:
    """[H, N, N] bias gathered from a [(2gh-1)(2gw-1), H] table."""
    table = np.asarray(table, dtype=np.float64)
    assert table.shape[0] == (2 * gh - 1) * (2 * gw - 1)
    idx = table_relative_index(gh, gw)
    return np.transpose(table[idx], (2, 0, 1))


def relpos_rows(qn: int, kn: int) -> np.ndarray:
    """Table row used by query coordinate qc and key coordinate kc -> [qn, kn].

    SAM blog, section "Bfloat16 half precision" (and the same passage of the
    Korean and Chinese write-ups): the image encoder scales the query and key
    coordinates (q_coords, k_coords) before they index the table.  Reading:
    the axis with fewer positions is stretched onto the other's range, so a
    query coordinate counts max(kn/qn, 1) units and a key coordinate
    max(qn/kn, 1) units; the row is the floor of the scaled difference,
    shifted by the largest scaled key coordinate so that it starts at 0:
    floor(qc*max(kn/qn,1) - kc*max(qn/kn,1) + (kn-1)*max(qn/kn,1)).
    Evaluated in exact rational arithmetic.  With qn == kn this is
    qc - kc + kn - 1, and every row lies in [0, 2*max(qn, kn) - 2].
    """
    sq = max(Fraction(kn, qn), Fraction(1))
    sk = max(Fraction(qn, kn), Fraction(1))
    out = np.empty((qn, kn), dtype=np.int64)
    for qc in range(qn):
        for kc in range(kn):
            out[qc, kc] = math.floor(qc * sq - kc * sk + (kn - 1) * sk)
    return out


def rel_pos_resized(table: np.ndarray, m: int) -> np.ndarray:
    """A relative-position table of L rows resized to m rows -> [m, d].

    SAM blog, section "Bfloat16 half precision" (and the same passage of the
    Korean and Chinese write-ups) names ``rel_pos_resized``: the table is
    resized when its length differs from the 2*max-1 rows the grids need, but
    the rule is not given.  Reading (the plainest one the rest supports):
    linear interpolation along the relative-offset axis with both ends
    aligned -- row r of the result is the old table at position
    p = r*(L-1)/(m-1), i.e. (1-f)*T[i] + f*T[i+1] with i = floor(p),
    f = p - i (a table of one row is repeated; m == 1 takes row 0).  It keeps
    the table unchanged when L == m, reproduces tables that are affine in the
    offset exactly, and keeps the end rows.  p is taken in exact rational
    arithmetic.
    """
    table = np.asarray(table, dtype=np.float64)
    L = table.shape[0]
    if L == m:
        return table.copy()
    out = np.empty((m,) + table.shape[1:])
    for r in range(m):
        if L == 1 or m == 1:
            out[r] = table[0]
            continue
        p = Fraction(r * (L - 1), m - 1)
        i = math.floor(p)
        f = float(p - i)
        out[r] = table[i] if i >= L - 1 else (1.0 - f) * table[i] + f * table[i + 1]
    return out


def e4m3_decode(codes) -> np.ndarray:
    """Values of 8-bit E4M3 floating-point codes -> float64 array.

    E4M3 as the OCP 8-bit floating point specification defines it: bit 7
    sign, bits 6..3 exponent e with bias 7, bits 2..0 mantissa m.  e > 0:
    (-1)^s * 2^(e-7) * (1 + m/8); e == 0: subnormal (-1)^s * 2^-6 * m/8.
    There are no infinities; the codes with e == 15 and m == 7 (0x7F, 0xFF)
    are NaN, so the largest finite magnitude is 2^8 * 1.75 = 448.
    """
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E4M3 codes are bytes 0..255")
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def dequantize_e4m3(codes, scale: float) -> np.ndarray:
    """code * scale in float64: the value an 8-bit input stands for, with its
    tensor's scale (see the low-precision reading in the module notes)."""
    return e4m3_decode(codes) * float(scale)


def relpos_bias(q_rows: np.ndarray, rows: np.ndarray, rh: np.ndarray,
                rw: np.ndarray, gh: int, gw: int, kgh: Optional[int] = None,
                kgw: Optional[int] = None) -> np.ndarray:
    """Decomposed relative-position bias for selected query rows -> [R, Nk].

    SAM blog, section "Bfloat16 half precision": per-query coordinates index
    the relative-position tables.  rel_h[i, kh] = q_i . Rh[row_h(qh_i, kh)]
    and rel_w[i, kw] = q_i . Rw[row_w(qw_i, kw)] (rows from
    :func:`relpos_rows`; on equal grids Rh[qh_i - kh + gh - 1]); the bias of
    key j = (kh, kw) of the kgh x kgw key grid is rel_h[i, kh] + rel_w[i, kw].
    Queries sit on the gh x gw grid; q is the raw query row.  Tables of
    another length than 2*max-1 rows are first resized to it
    (:func:`rel_pos_resized`).
    """
    kgh = gh if kgh is None else kgh
    kgw = gw if kgw is None else kgw
    q_rows = np.asarray(q_rows, dtype=np.float64)
    rh = rel_pos_resized(rh, 2 * max(gh, kgh) - 1)
    rw = rel_pos_resized(rw, 2 * max(gw, kgw) - 1)
    qh, qw = np.asarray(rows) // gw, np.asarray(rows) % gw
    rh_sel = rh[relpos_rows(gh, kgh)[qh]]                    # [R, kgh, d]
    rw_sel = rw[relpos_rows(gw, kgw)[qw]]                    # [R, kgw, d]
    rel_h = np.einsum("rc,rkc->rk", q_rows, rh_sel)          # [R, kgh]
    rel_w = np.einsum("rc,rkc->rk", q_rows, rw_sel)          # [R, kgw]
    return (rel_h[:, :, None] + rel_w[:, None, :]).reshape(len(rows), kgh * kgw)


def relpos_bias_gather(q_rows: np.ndarray, rows: np.ndarray, rh: np.ndarray,
                       rw: np.ndarray, gh: int, gw: int) -> np.ndarray:
    """Same bias through the literal per-pair gather (small equal grids only).

    For every (query i, key j) pair the two table rows are gathered first,
    [R, N, d], and then dotted with q_i: q_i . Rh[dh] + q_i . Rw[dw].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    rh = np.asarray(rh, dtype=np.float64)
    rw = np.asarray(rw, dtype=np.float64)
    qr, qc = np.asarray(rows) // gw, np.asarray(rows) % gw
    kr, kc = token_coords(gh, gw)
    gath_h = rh[qr[:, None] - kr[None, :] + gh - 1]          # [R, N, d]
    gath_w = rw[qc[:, None] - kc[None, :] + gw - 1]          # [R, N, d]
    return (np.einsum("rc,rjc->rj", q_rows, gath_h)
            + np.einsum("rc,rjc->rj", q_rows, gath_w))


# ---------------------------------------------------------------------------
# Windows, the cyclic shift and the shifted-region mask
# ---------------------------------------------------------------------------

def shift_region_labels(img_h: int, img_w: int, win_h: int, win_w: int,
                        shift_h: int, shift_w: int) -> np.ndarray:
    """[img_h, img_w] region id of every pixel of the shifted image.

    Swin talk, section 1: the window shift brings pixels from different parts
    of the image into one window; pairs from different parts are kept apart.
    Each axis splits into the three ranges [0, n-win), [n-win, n-shift),
    [n-shift, n); regions are numbered row range major.
    """
    labels = np.zeros((img_h, img_w), dtype=np.int64)
    hs = [(0, img_h - win_h), (img_h - win_h, img_h - shift_h), (img_h - shift_h, img_h)]
    ws = [(0, img_w - win_w), (img_w - win_w, img_w - shift_w), (img_w - shift_w, img_w)]
    cnt = 0
    for (h0, h1) in hs:
        for (w0, w1) in ws:
            labels[h0:h1, w0:w1] = cnt
            cnt += 1
    return labels


def window_partition(x: np.ndarray, win_h: int, win_w: int) -> np.ndarray:
    """[B, H, img_h, img_w, d] -> [B * nW, H, win_h*win_w, d].

    Windows row-major inside an image, images outermost, tokens row-major
    inside a window (Swin talk, section 1: the image is split into windows and
    attention runs inside each window only).
    """
    B, H, ih, iw, d = x.shape
    nwy, nwx = ih // win_h, iw // win_w
    assert nwy * win_h == ih and nwx * win_w == iw
    y = x.reshape(B, H, nwy, win_h, nwx, win_w, d)
    y = y.transpose(0, 2, 4, 1, 3, 5, 6)                      # B, wy, wx, H, th, tw, d
    return y.reshape(B * nwy * nwx, H, win_h * win_w, d)


def window_reverse(w: np.ndarray, img_h: int, img_w: int, win_h: int,
                   win_w: int) -> np.ndarray:
    """Inverse of :func:`window_partition`."""
    nwy, nwx = img_h // win_h, img_w // win_w
    BnW, H, N, d = w.shape
    B = BnW // (nwy * nwx)
    y = w.reshape(B, nwy, nwx, H, win_h, win_w, d)
    y = y.transpose(0, 3, 1, 4, 2, 5, 6)                      # B, H, wy, th, wx, tw, d
    return y.reshape(B, H, img_h, img_w, d)


def padded_extent(n: int, win: int) -> int:
    """Image side padded up to a whole number of windows."""
    return -(-n // win) * win


def shift_mask(img_h: int, img_w: int, win_h: int, win_w: int, shift_h: int,
               shift_w: int, value: float = -100.0) -> np.ndarray:
    """[nW, N, N] additive mask: ``value`` where query and key regions differ
    (regions of the image padded to whole windows)."""
    ph, pw = padded_extent(img_h, win_h), padded_extent(img_w, win_w)
    labels = shift_region_labels(ph, pw, win_h, win_w, shift_h, shift_w)
    lw = window_partition(labels[None, None, :, :, None].astype(np.float64),
                          win_h, win_w)[:, 0, :, 0]           # [nW, N]
    diff = lw[:, :, None] != lw[:, None, :]
    return np.where(diff, float(value), 0.0)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _additive_rows(b: int, h: int, rows: np.ndarray, q_rows: np.ndarray,
                   Nk: int, bias: Bias, mask: Mask, cache: dict) -> np.ndarray:
    """bias + mask for query rows ``rows`` of batch item b, head h -> [R, Nk]."""
    add = np.zeros((len(rows), Nk), dtype=np.float64)
    if bias is not None and bias.kind != "none":
        if bias.kind == "table":
            gh, gw = bias.grid
            key = ("table", h)
            if key not in cache:
                cache[key] = table_bias(bias.table, gh, gw)[h]
            add += cache[key][rows]
        elif bias.kind == "relpos":
            gh, gw = bias.grid
            kgh, kgw = bias.kgrid if bias.kgrid is not None else (gh, gw)
            add += relpos_bias(q_rows, rows, bias.rh, bias.rw, gh, gw, kgh, kgw)
        elif bias.kind == "additive":
            a = np.asarray(bias.add, dtype=np.float64)
            add += a[b % a.shape[0]][rows]
        else:
            raise ValueError(f"unknown bias kind {bias.kind!r}")
    if mask is not None and mask.kind != "none":
        if mask.kind == "shift":
            if "shift" not in cache:
                cache["shift"] = shift_mask(*mask.window, value=mask.value)
            m = cache["shift"]
            add += m[b % m.shape[0]][rows]
        elif mask.kind == "additive":
            a = np.asarray(mask.add, dtype=np.float64)
            add += a[b % a.shape[0]][rows]
        else:
            raise ValueError(f"unknown mask kind {mask.kind!r}")
    return add


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax exp(s - max) / sum, in float64."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_probs(q, k, bias: Optional[Bias] = None,
                    mask: Optional[Mask] = None) -> np.ndarray:
    """Attention map P = softmax(scale*QK^T + bias + mask), [B, H, Nq, Nk]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    scale = 1.0 / np.sqrt(d)
    cache: dict = {}
    out = np.empty((B, H, Nq, Nk))
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            s = s + _additive_rows(b, h, rows, q[b, h], Nk, bias, mask, cache)
            out[b, h] = _softmax_rows(s)
    return out


def attention_logsumexp(q, k, bias: Optional[Bias] = None,
                        mask: Optional[Mask] = None) -> np.ndarray:
    """Per-row log-sum-exp of the logits, [B, H, Nq]:
    L_i = log sum_j exp(scale * q_i.k_j + bias_ij + mask_ij) (natural log).

    The normaliser of the softmax rows of :func:`attention_probs`
    (P_ij = exp(s_ij - L_i)); an attention kernel can report it so that a
    backward pass recomputes P without a pass of its own over the keys.
    Computed as max + log(sum(exp(s - max))) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    scale = 1.0 / np.sqrt(d)
    cache: dict = {}
    out = np.empty((B, H, Nq))
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T) + _additive_rows(b, h, rows, q[b, h], Nk, bias, mask, cache)
            m = s.max(axis=-1)
            out[b, h] = m + np.log(np.exp(s - m[:, None]).sum(axis=-1))
    return out


def attention(q, k, v, bias: Optional[Bias] = None, mask: Optional[Mask] = None,
              select: Optional[Sequence] = None, row_block: int = 512):
    """O = softmax(scale*QK^T + bias + mask) V in float64.

    q: [B, H, Nq, d]; k, v: [B, H, Nk, d] (batched layout: windows are extra
    batch items).  With ``select`` = [(b, h, rows), ...] only those output
    rows are computed and a list of [len(rows), d] arrays is returned;
    otherwise the full [B, H, Nq, d] output.  Query rows are processed in
    blocks of ``row_block``; each row's softmax is independent, so this is
    still the plain definition.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    assert k.shape == (B, H, Nk, d) and v.shape == (B, H, Nk, v.shape[3])
    scale = 1.0 / np.sqrt(d)
    cache: dict = {}

    def rows_out(b, h, rows):
        rows = np.asarray(rows)
        res = np.empty((len(rows), v.shape[3]))
        for s0 in range(0, len(rows), row_block):
            r = rows[s0:s0 + row_block]
            s = scale * (q[b, h, r] @ k[b, h].T)
            s = s + _additive_rows(b, h, r, q[b, h, r], Nk, bias, mask, cache)
            res[s0:s0 + row_block] = _softmax_rows(s) @ v[b, h]
        return res

    if select is not None:
        return [rows_out(b, h, rows) for (b, h, rows) in select]
    out = np.empty((B, H, Nq, v.shape[3]))
    all_rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            out[b, h] = rows_out(b, h, all_rows)
    return out


def attention_image(q, k, v, window: tuple, bias: Optional[Bias] = None,
                    mask: Optional[Mask] = None) -> np.ndarray:
    """Shifted-window attention on image-layout tensors [B, H, img_h*img_w, d].

    Swin talk, section 2: shift, partition, attention, reverse partition and
    reverse shift.  The image is zero-padded at the bottom and right to whole
    windows, the content is rolled by (-sh, -sw), partitioned into windows,
    attended with the window bias and mask, merged back, rolled by (+sh, +sw)
    and cropped to the image.
    """
    img_h, img_w, win_h, win_w, sh, sw = window
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    assert N == img_h * img_w
    ph, pw = padded_extent(img_h, win_h), padded_extent(img_w, win_w)

    def to_windows(x):
        x = x.reshape(B, H, img_h, img_w, x.shape[-1])
        x = np.pad(x, ((0, 0), (0, 0), (0, ph - img_h), (0, pw - img_w), (0, 0)))
        x = np.roll(x, shift=(-sh, -sw), axis=(2, 3))
        return window_partition(x, win_h, win_w)

    ow = attention(to_windows(q), to_windows(k), to_windows(v), bias, mask)
    o = window_reverse(ow, ph, pw, win_h, win_w)
    o = np.roll(o, shift=(sh, sw), axis=(2, 3))[:, :, :img_h, :img_w]
    return o.reshape(B, H, N, v.shape[-1])


def attention_image_logsumexp(q, k, window: tuple, bias: Optional[Bias] = None,
                              mask: Optional[Mask] = None) -> np.ndarray:
    """Per-token log-sum-exp of the shifted-window attention in image order,
    [B, H, img_h*img_w]: the windows' :func:`attention_logsumexp`, mapped back
    through the reverse partition, reverse shift and crop of
    :func:`attention_image`."""
    img_h, img_w, win_h, win_w, sh, sw = window
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, d = q.shape
    ph, pw = padded_extent(img_h, win_h), padded_extent(img_w, win_w)

    def to_windows(x):
        x = x.reshape(B, H, img_h, img_w, x.shape[-1])
        x = np.pad(x, ((0, 0), (0, 0), (0, ph - img_h), (0, pw - img_w), (0, 0)))
        x = np.roll(x, shift=(-sh, -sw), axis=(2, 3))
        return window_partition(x, win_h, win_w)

    lw = attention_logsumexp(to_windows(q), to_windows(k), bias, mask)[..., None]
    lo = window_reverse(lw, ph, pw, win_h, win_w)
    lo = np.roll(lo, shift=(sh, sw), axis=(2, 3))[:, :, :img_h, :img_w]
    return lo.reshape(B, H, N)


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------

def attention_backward(q, k, v, dout, bias: Optional[Bias] = None,
                       mask: Optional[Mask] = None) -> dict:
    """Gradients of L = sum(dout * O) for O = softmax(scale*QK^T + B + M) V.

    The Swin talk, section 2, trains with a fused window op that has its own
    backward; the gradients here are the plain chain rule of the forward
    definition, written out per (batch item, head) in float64:
      P = softmax rows of S,  dV = P^T dO,  dP = dO V^T,
      dS = P * (dP - rowsum(P * dP)),
      dQ = scale * dS K,  dK = scale * dS^T Q,
      d_table[r, h] = sum of dS over the pairs (i, j) of head h that read
                      table row r (summed over batch items),
      decomposed relative position: the bias is rel_h[i, kh] + rel_w[i, kw]
      with rel_h[i, kh] = q_i . Rh[row_h(qh_i, kh)] (SAM blog, section
      "Bfloat16 half precision"; see relpos_bias), so through that
      decomposition
        dRelH[i, kh] = sum over kw of dS[i, (kh, kw)],
        dRelW[i, kw] = sum over kh of dS[i, (kh, kw)],
        dQ_i += sum_kh dRelH[i, kh] Rh[row_h(qh_i, kh)]
                + sum_kw dRelW[i, kw] Rw[row_w(qw_i, kw)],
        dRh[m] = sum of dRelH[i, kh] q_i over (b, h, i, kh) with
                 row_h(qh_i, kh) = m (dRw likewise),
      for the tables of the needed length, then mapped to the stored tables
      through the transpose of the resize.
    The mask is a constant and has no gradient.  Returns dq, dk, dv and,
    with a table bias, dtable [(2gh-1)(2gw-1), H]; with the relative
    position, drh, drw.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    scale = 1.0 / np.sqrt(d)
    cache: dict = {}
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    res = {}
    if bias is not None and bias.kind == "table":
        gh, gw = bias.grid
        idx = table_relative_index(gh, gw)
        dtable = np.zeros((idx.max() + 1, H))
    if bias is not None and bias.kind == "relpos":
        gh, gw = bias.grid
        kgh, kgw = bias.kgrid if bias.kgrid is not None else (gh, gw)
        rh = rel_pos_resized(bias.rh, 2 * max(gh, kgh) - 1)
        rw = rel_pos_resized(bias.rw, 2 * max(gw, kgw) - 1)
        row_h = relpos_rows(gh, kgh)[np.arange(Nq) // gw]    # [Nq, kgh]: table row of (query, kh)
        row_w = relpos_rows(gw, kgw)[np.arange(Nq) % gw]     # [Nq, kgw]
        drh, drw = np.zeros_like(rh), np.zeros_like(rw)
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            s = s + _additive_rows(b, h, rows, q[b, h], Nk, bias, mask, cache)
            p = _softmax_rows(s)
            dv[b, h] = p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, h].T
            ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
            if bias is not None and bias.kind == "table":
                np.add.at(dtable[:, h], idx, ds)
            if bias is not None and bias.kind == "relpos":
                ds3 = ds.reshape(Nq, kgh, kgw)
                d_relh, d_relw = ds3.sum(axis=2), ds3.sum(axis=1)     # [Nq, kgh], [Nq, kgw]
                dq[b, h] += (np.einsum("ik,ikc->ic", d_relh, rh[row_h])
                             + np.einsum("ik,ikc->ic", d_relw, rw[row_w]))
                np.add.at(drh, row_h, d_relh[:, :, None] * q[b, h][:, None, :])
                np.add.at(drw, row_w, d_relw[:, :, None] * q[b, h][:, None, :])
    res.update(dq=dq, dk=dk, dv=dv)
    if bias is not None and bias.kind == "table":
        res["dtable"] = dtable
    if bias is not None and bias.kind == "relpos":
        # Gradients of the stored tables: the resize is linear, T' = W T with
        # W the resize of the identity, so dT = W^T dT'.
        wh = rel_pos_resized(np.eye(np.asarray(bias.rh).shape[0]), rh.shape[0])
        ww = rel_pos_resized(np.eye(np.asarray(bias.rw).shape[0]), rw.shape[0])
        res["drh"], res["drw"] = wh.T @ drh, ww.T @ drw
    return res


def attention_image_backward(q, k, v, dout, window: tuple, bias: Optional[Bias] = None,
                             mask: Optional[Mask] = None) -> dict:
    """Gradients of the shifted-window attention on image-layout tensors: the
    padding, roll and partition of :func:`attention_image` are index maps, so
    the gradients are mapped back through the same maps (padding rows
    dropped)."""
    img_h, img_w, win_h, win_w, sh, sw = window
    B, H, N, d = np.asarray(q).shape
    ph, pw = padded_extent(img_h, win_h), padded_extent(img_w, win_w)

    def to_windows(x):
        x = np.asarray(x, dtype=np.float64).reshape(B, H, img_h, img_w, x.shape[-1])
        x = np.pad(x, ((0, 0), (0, 0), (0, ph - img_h), (0, pw - img_w), (0, 0)))
        x = np.roll(x, shift=(-sh, -sw), axis=(2, 3))
        return window_partition(x, win_h, win_w)

    def from_windows(g):
        x = window_reverse(g, ph, pw, win_h, win_w)
        x = np.roll(x, shift=(sh, sw), axis=(2, 3))[:, :, :img_h, :img_w]
        return x.reshape(B, H, N, g.shape[-1])

    res = attention_backward(to_windows(q), to_windows(k), to_windows(v), to_windows(dout), bias, mask)
    for key in ("dq", "dk", "dv"):
        res[key] = from_windows(res[key])
    return res


def _dequantized(w, arrays: dict) -> dict:
    """``arrays`` with q, k, v dequantized when workload ``w`` stores them as
    E4M3 codes (attribute ``qkv`` == "e4m3"; ``arrays["descale"]`` holds the
    scales of q, k and v in that order)."""
    if getattr(w, "qkv", "same") != "e4m3":
        return arrays
    s = np.asarray(arrays["descale"], dtype=np.float64).reshape(-1)
    out = dict(arrays)
    for i, name in enumerate(("q", "k", "v")):
        out[name] = dequantize_e4m3(arrays[name], s[i])
    return out


def _workload_terms(w, arrays: dict):
    """The Bias and Mask of a workload record, tables taken from ``arrays``."""
    bias = Bias("none")
    if w.bias == "table":
        bias = Bias("table", grid=w.grid, table=arrays["table"])
    elif w.bias == "relpos":
        bias = Bias("relpos", grid=w.grid, kgrid=getattr(w, "kgrid", None), rh=arrays["rh"],
                    rw=arrays["rw"])
    elif w.bias == "additive":
        bias = Bias("additive", add=arrays["bias_add"])
    mask = Mask("none")
    if w.mask == "shift":
        mask = Mask("shift", window=tuple(w.window))
    elif w.mask == "additive":
        mask = Mask("additive", add=arrays["mask_add"])
    return bias, mask


def run_workload(w, arrays: dict, select: Optional[Sequence] = None):
    """Oracle output for a workload description.

    ``w`` is any object with the attributes bias, grid, mask, layout, window
    (a workload record); ``arrays`` maps q, k, v and the bias tables
    (table / rh, rw / bias_add, mask_add) to float64 numpy arrays holding the
    exact device values.  ``select`` as in :func:`attention` (batched layout).
    """
    arrays = _dequantized(w, arrays)
    bias, mask = _workload_terms(w, arrays)
    if w.layout == "image":
        assert select is None, "image layout is evaluated whole"
        return attention_image(arrays["q"], arrays["k"], arrays["v"], tuple(w.window), bias, mask)
    return attention(arrays["q"], arrays["k"], arrays["v"], bias, mask, select=select)


def run_workload_logsumexp(w, arrays: dict) -> np.ndarray:
    """Oracle per-row log-sum-exp for a workload description (see
    run_workload): [B, H, Nq], in image order for the image layout."""
    arrays = _dequantized(w, arrays)
    bias, mask = _workload_terms(w, arrays)
    if w.layout == "image":
        return attention_image_logsumexp(arrays["q"], arrays["k"], tuple(w.window), bias, mask)
    return attention_logsumexp(arrays["q"], arrays["k"], bias, mask)


def run_workload_backward(w, arrays: dict) -> dict:
    """Oracle gradients for a workload description (see run_workload);
    ``arrays`` also holds ``dout``, the gradient of the output."""
    bias, mask = _workload_terms(w, arrays)
    if w.layout == "image":
        return attention_image_backward(arrays["q"], arrays["k"], arrays["v"], arrays["dout"],
                                        tuple(w.window), bias, mask)
    return attention_backward(arrays["q"], arrays["k"], arrays["v"], arrays["dout"], bias, mask)
