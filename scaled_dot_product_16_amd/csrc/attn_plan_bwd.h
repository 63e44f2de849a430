// Geometry, LDS and workspace of the backward kernels, and their plan, in
// plain C++ like the forward's (attn_plan.h includes this file at its end):
// the window backward (attn_bwd_win) and the tiled row / column kernels
// (attn_bwd_rows, attn_bwd_cols) with their relative-position forms.
#ifndef ATTN_PLAN_BWD_H_
#define ATTN_PLAN_BWD_H_

#include "attn_plan.h"

namespace attn {

// Window backward kernel (attn_bwd_win): Q, K, V and dO tiles of 64 rows
// (head dim padded to the 32-wide contraction), P^T and dS^T in the element
// type (64 keys x 64 queries, rows padded by 8), the per-key lookup parts
// and the table.  (A pad of 16, which the tiled backward takes, measured 2 %
// slower here.)  With a TABLE bias, dS^T is also kept in fp32 for the table
// gradient ([Nk][Nq + 1] floats): written after the K and V tiles are dead,
// into their space when it fits there, else after the table.
template <int D>
struct WinBwdCfg {
  static constexpr int NT = kWinWaves * 64;
  static constexpr int KCH = (D + 31) / 32;
  static constexpr int DK = KCH * 32;
  static constexpr int CBD = (D + 15) / 16;   // 16-wide blocks of dQ, dK, dV columns
  static constexpr int ROW = DK + 8;
  static constexpr int PROW = 64 + 8;
  static constexpr int RCH = D / 8;
  static constexpr int NCH = 64 * RCH;
  static constexpr int CPT = (NCH + NT - 1) / NT;
  static constexpr size_t KV_BYTES = (size_t)2 * 64 * ROW * 2;  // the K and V tiles
  static constexpr size_t BYTES = (size_t)4 * 64 * ROW * 2 + (size_t)2 * 64 * PROW * 2 + 64 * 4;
};

constexpr size_t win_bwd_sf_bytes(const AttnArgs& a) {
  return a.bias_kind == ATTN_BIAS_TABLE ? (size_t)a.Nk * (a.Nq + 1) * 4 : 0;
}
template <int D>
constexpr bool win_bwd_sf_in_kv(const AttnArgs& a) {
  return win_bwd_sf_bytes(a) <= WinBwdCfg<D>::KV_BYTES;
}
template <int D>
constexpr size_t win_bwd_lds_bytes(const AttnArgs& a) {
  const size_t n = WinBwdCfg<D>::BYTES + (win_uses_table(a) ? (size_t)9 * win_tab_entries(a) * 4 : 0);
  return n + (win_bwd_sf_in_kv<D>(a) ? 0 : win_bwd_sf_bytes(a));
}

// ---------------------------------------------------------------------------
// Tiled backward (attn_bwd_rows / attn_bwd_cols) geometry
// ---------------------------------------------------------------------------

// The staged tiles are read both ways: 16-byte row reads for S and dP, and
// transposing reads for dQ, dK, dV.  Rows padded by 16 elements past the
// 32-multiple contraction width have a stride of 8 or 24 dwords modulo 32,
// which keeps the transposing reads' 4 rows on distinct banks; a pad of 8
// puts them two to a bank (measured 7 % slower on SD self-attention and SAM
// global backward).
constexpr int kBwdRowPad = 16;

// Relative-position forms of the tiled backward: none; general grids (the
// row kernel keeps per-lane private sums of dRelH/dRelW in LDS, 1280 bytes
// per column of gh + gw, so gh + gw <= kBwdRelMaxCols, and at d = 80, where
// the staged tiles are larger, gh + gw <= 83); 64-wide grids
// (a 64-key tile is one grid row: dRelH is a row sum per tile, dRelW and
// rel_w stay in registers per key slot); small general grids (gh + gw <=
// 32, at most 256 keys: the row kernel adds the bias and gathers dRelH /
// dRelW on the matrix cores through a one-hot table of the keys' grid
// positions, E[key][x] = 1 for x = kh and x = gh + kw; its column kernel is
// the general form's).
constexpr int kBwdRelNone = 0, kBwdRelGeneral = 1, kBwdRelRow64 = 2, kBwdRelAug = 3;
constexpr int kBwdRelMaxCols = 84;
constexpr int kBwdAugMaxCols = 32, kBwdAugMaxKeys = 256;
// Row stride (elements) of the one-hot key table: 32 columns plus the pad
// that keeps its transposing reads on distinct banks.
constexpr int kBwdAugRow = 32 + kBwdRowPad;
// Small general grids hand each query's rel_h / rel_w row to the column
// kernel as 32 columns / scale in the element type, high then low part
// (64 elements, 128 bytes); the column kernel stages a query tile of them
// with rows of kBwdAugQRow elements.
constexpr int kBwdAugQRow = 64 + kBwdRowPad;

constexpr int bwd_rel_mode(const AttnArgs& a) {
  return a.bias_kind != ATTN_BIAS_RELPOS ? kBwdRelNone
         : (a.gw == 64 && a.gh <= 64)     ? kBwdRelRow64
         : (a.gh + a.gw <= kBwdAugMaxCols && a.Nk <= kBwdAugMaxKeys) ? kBwdRelAug
                                                                       : kBwdRelGeneral;
}
// General grids in either form: rel_h / rel_w rows of the workgroup's
// queries in LDS, and all columns staged by the column kernel.
constexpr bool bwd_rel_general(int mode) { return mode == kBwdRelGeneral || mode == kBwdRelAug; }

// Rows of the stacked table [Rh; Rw] (equal grids, tables of the needed length).
constexpr int bwd_rel_rows(const AttnArgs& a) { return 2 * a.gh - 1 + 2 * a.gw - 1; }

// Per-workgroup slot of the partial table gradients (floats): the [dRh; dRw]
// part, and in the 64-wide form first the workgroup's dRelH^T and dRelW^T
// ([gh + 64][64] floats, read back after the key loop).
constexpr size_t bwd_part_stride(const AttnArgs& a) {
  const size_t part = (size_t)bwd_rel_rows(a) * (size_t)a.D;
  const size_t drel = bwd_rel_mode(a) == kBwdRelRow64 ? (size_t)(a.gh + 64) * 64 : 0;
  return part > drel ? part : drel;
}
// Workspace of the tiled backward, in floats: the rows' L and D (B*H*Nq
// each), then with the relative position the rel_h / rel_w rows of every
// query ([B*H][gh + gw][Nq] floats, or [B*H][Nq][64] elements in the one-
// hot table's form, 32 floats a query; written by the row kernel, read by
// the column kernel) and one partial slot per row-kernel workgroup
// ([B*H*ceil(Nq/64)] slots of pstride floats, summed in a fixed order
// afterwards).
struct BwdWs {
  size_t L, D, rel, part, pstride, total;
};
constexpr BwdWs bwd_ws_layout(const AttnArgs& a) {
  const size_t n = (size_t)a.B * a.H * a.Nq;
  BwdWs w{0, n, 0, 0, 0, 0};
  size_t off = (2 * n + 3) / 4 * 4;
  w.rel = off;
  if (a.bias_kind == ATTN_BIAS_RELPOS) {
    const size_t per_q = bwd_rel_mode(a) == kBwdRelAug ? 32 : (size_t)(a.gh + a.gw);
    off = (off + n * per_q + 3) / 4 * 4;
    w.part = off;
    w.pstride = bwd_part_stride(a);
    off += (size_t)a.B * a.H * (size_t)((a.Nq + 63) / 64) * w.pstride;
  } else {
    w.part = off;
  }
  w.total = off;
  return w;
}

// LDS of the row kernel: the K/V stages, used after the key loop for the
// coefficient matrix A of the table-gradient products ([bwd_rel_arows][
// kBwdARow] elements; a row stride of 40 dwords keeps the transposing reads
// of A on distinct banks); then the relative-position region.  General
// grids: rel_h/rel_w (later dRel, one staged table, the Q tile) and the
// per-lane dRel sums.  The 64-wide form keeps rel_h in the workspace and
// dRelH / dRelW in the workgroup's partial slot, so its region only holds a
// 64-row slice of a table, then the Q tile: 51 KB at d <= 64, three
// workgroups per CU.
constexpr int kBwdARow = 80;
constexpr int bwd_up32(int n) { return (n + 31) / 32 * 32; }
// Rows of A: each table's rows padded to 32 for the dQ products (Rh rows
// from 0, Rw rows from 2gh-1) and all rows padded to 16 for the partial.
constexpr int bwd_rel_arows(const AttnArgs& a) {
  const int rh = 2 * a.gh - 1, rw = 2 * a.gw - 1;
  const int x = bwd_up32(rh) > rh + bwd_up32(rw) ? bwd_up32(rh) : rh + bwd_up32(rw);
  const int y = (rh + rw + 15) / 16 * 16;
  return x > y ? x : y;
}
// Rows of one staged table slice for the dQ products: a whole table
// padded to 32 rows (general grids), or 64 rows at a time (64-wide form).
constexpr int bwd_rel_tab_rows(const AttnArgs& a) {
  if (bwd_rel_mode(a) == kBwdRelRow64) return 64;
  const int rh = bwd_up32(2 * a.gh - 1), rw = bwd_up32(2 * a.gw - 1);
  return rh > rw ? rh : rw;
}
// Row stride of a staged table slice (elements): CBD*16 columns plus the
// transposing-read pad.
template <int D>
constexpr int bwd_rel_tab_row() {
  return (D + 15) / 16 * 16 + v_row_pad((D + 15) / 16 * 16);
}
template <int D>
constexpr size_t bwd_rel_tab_bytes(const AttnArgs& a) {
  return (size_t)bwd_rel_tab_rows(a) * bwd_rel_tab_row<D>() * 2;
}
template <int D>
constexpr size_t bwd_stage_bytes(const AttnArgs& a) {
  constexpr int ROW = (D + 31) / 32 * 32 + kBwdRowPad;
  size_t s = (size_t)4 * 64 * ROW * 2;
  if (a.bias_kind == ATTN_BIAS_RELPOS) {
    const size_t am = (size_t)bwd_rel_arows(a) * kBwdARow * 2;
    s = s > am ? s : am;
    // 64-wide form: the prologue's G_w[128][64] floats.
    if (bwd_rel_mode(a) == kBwdRelRow64 && s < (size_t)128 * 64 * 4) s = (size_t)128 * 64 * 4;
  }
  return (s + 15) / 16 * 16;
}
// Bytes at the end of the relative-position region that only the key loop
// uses: the per-lane dRel sums (general grids) or the one-hot key table
// (small general grids, one row per key of the padded tiles).
constexpr size_t bwd_rows_acc_bytes(const AttnArgs& a) {
  const int mode = bwd_rel_mode(a);
  if (mode == kBwdRelGeneral) return (size_t)256 * ((a.gh + a.gw) | 1) * 4;
  if (mode == kBwdRelAug) return (size_t)((a.Nk + 63) / 64 * 64) * kBwdAugRow * 2;
  return 0;
}
template <int D>
constexpr size_t bwd_rows_rel_bytes(const AttnArgs& a) {
  constexpr int ROW = (D + 31) / 32 * 32 + kBwdRowPad;
  const int mode = bwd_rel_mode(a);
  if (mode == kBwdRelNone) return 0;
  const size_t g = (size_t)(a.gh + a.gw);
  size_t rel = bwd_rel_general(mode) ? 64 * g * 4 : 0;
  const size_t qt = (size_t)64 * ROW * 2;
  rel = (rel > qt ? rel : qt);
  const size_t acc = bwd_rows_acc_bytes(a), tab = bwd_rel_tab_bytes<D>(a);
  if (rel + acc < tab) rel = tab - acc;
  rel = (rel + 15) / 16 * 16;
  return rel + acc;
}
// Columns of rel_h / rel_w the column kernel stages per query tile: all of
// them for general grids; none in the 64-wide form (the key tile's rel_h
// column joins the staged log-sum-exp, and each lane reads its own rel_w
// column from the workspace) or the one-hot table's form (which stages the
// packed rows instead).
constexpr int bwd_cols_rel_cols(const AttnArgs& a) {
  return bwd_rel_mode(a) == kBwdRelGeneral ? a.gh + a.gw : 0;
}
// Bytes of the column kernel's two stages of relative-position data.
constexpr size_t bwd_cols_rel_bytes(const AttnArgs& a) {
  return bwd_rel_mode(a) == kBwdRelAug ? (size_t)2 * 64 * kBwdAugQRow * 2
                                       : (size_t)2 * 64 * bwd_cols_rel_cols(a) * 4;
}

// The backward of a validated call (half precision): window units (at most
// 64 queries and keys; any bias but the relative position, any mask), or
// the tiled row/column kernels for longer sequences in the batched layout
// without a mask and with no bias or the relative position (equal grids,
// tables of the needed length).  blocks: the larger of the two tiled grids;
// rmode: the relative-position form.
template <int D>
inline Plan plan_bwd_half(const AttnArgs& a) {
  Plan p{};
  p.hg = 1;
  p.nw = kWinWaves;
  if (a.Nq <= 64 && a.Nk <= 64 && a.bias_kind != ATTN_BIAS_RELPOS) {
    p.kernel = kKernWin;
    p.blocks = (int64_t)a.B * a.H;
    p.lds = win_bwd_lds_bytes<D>(a);
    return p;
  }
  const bool rel_ok = a.bias_kind == ATTN_BIAS_RELPOS && a.gh == a.kgh && a.gw == a.kgw &&
                      !relpos_resized(a) &&
                      (bwd_rel_mode(a) == kBwdRelRow64 || a.gh + a.gw <= kBwdRelMaxCols);
  if ((a.bias_kind != ATTN_BIAS_NONE && !rel_ok) || a.mask_kind != ATTN_MASK_NONE || a.image) {
    p.kernel = -1;
    return p;
  }
  constexpr int ROW = (D + 31) / 32 * 32 + kBwdRowPad;
  p.kernel = kKernMfma;
  p.rmode = bwd_rel_mode(a);
  p.bm = 64;
  const int64_t nt = (a.Nq > a.Nk ? a.Nq : a.Nk) + 63;
  p.blocks = nt / 64 * a.H * a.B;
  // Row kernel: two LDS stages of the K and V tiles (and the relative-
  // position regions); column kernel: two stages of the Q and dO tiles, of
  // the 64 rows' L and D, and of the staged rel_h / rel_w columns.
  const size_t rows = bwd_stage_bytes<D>(a) + bwd_rows_rel_bytes<D>(a);
  const size_t cols = (size_t)4 * 64 * ROW * 2 + 4 * 64 * 4 + bwd_cols_rel_bytes(a);
  p.lds = rows > cols ? rows : cols;
  return p;
}

// Workspace bytes of the backward: per-unit table gradients (window path
// with a table bias) or the tiled path's (bwd_ws_layout).
constexpr size_t bwd_workspace_bytes(const AttnArgs& a, int kernel) {
  if (kernel == kKernWin)
    return a.bias_kind == ATTN_BIAS_TABLE
               ? (size_t)a.B * a.H * (size_t)((2 * a.gh - 1) * (2 * a.gw - 1)) * 4
               : 0;
  return bwd_ws_layout(a).total * 4;
}

inline int make_bwd_plan(const AttnArgs& a, Plan* p) {
  if (a.dtype == ATTN_F32) return ATTN_E_UNSUPPORTED;
  switch (a.D) {
    case 32: *p = plan_bwd_half<32>(a); break;
    case 40: *p = plan_bwd_half<40>(a); break;
    case 64: *p = plan_bwd_half<64>(a); break;
    case 80: *p = plan_bwd_half<80>(a); break;
    default: return ATTN_E_UNSUPPORTED;
  }
  if (p->kernel < 0 || p->lds > kMaxLds || p->blocks > 0x7fffffff) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace attn

#endif  // ATTN_PLAN_BWD_H_
