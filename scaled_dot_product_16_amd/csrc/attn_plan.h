// Kernel choice and on-chip memory of a validated call, in plain C++ (no HIP
// headers): the host validation uses it, so attn_check reports the same
// status attn_fwd returns when a call's tiles or tables do not fit in LDS,
// and the launcher launches exactly what it says.  The tile geometry
// (MfmaCfg, WinCfg, ...) lives here for the same reason: the kernels and the
// byte counts below read the same constants.
//
// constexpr functions are usable from device code as well (clang treats
// them as host and device), so the kernels call the same helpers.
#ifndef ATTN_PLAN_H_
#define ATTN_PLAN_H_

#include <stddef.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace attn {

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// ---------------------------------------------------------------------------
// Tiled kernel (attn_fwd_mfma) geometry
// ---------------------------------------------------------------------------
constexpr int kNQB = 2;         // 16-query blocks per wave
constexpr int kKPad = 16;       // K tile row padding (elements; 16 measured faster than 8 and 24)
constexpr bool kOnesRow = true; // row sums from a ones row of V on the matrix cores

// V tile rows are padded to 16 elements past a multiple of 32 (row stride
// of 8 or 24 dwords modulo 32): the transposing reads then fetch the 4 rows
// x 4 column slices of each 16-lane group from distinct banks (also for 64
// banks with 32 lanes per pass).
constexpr int v_row_pad(int dv) { return ((16 - dv % 32) + 32) % 32; }

// Relative-position modes (forms) of the tiled kernel.
constexpr int kRelTables = 0;  // per-score lookups in LDS tables (also non-relpos biases)
constexpr int kRelRow64 = 1;   // 64-wide grids: Rw term seeds the accumulator, Rh term per row
constexpr int kRelAug = 2;     // gh + gw <= 32: bias folded into the QK^T contraction
constexpr int kTwoTiles = 3;   // no bias or mask, BN < Nk <= 2 BN: both key tiles loaded up front

template <int D, int NW, int NQB, bool AUG = false>
struct MfmaCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * NQB * 16;
  static constexpr int BN = 64;
  static constexpr int KCH = (D + 31) / 32;  // 32-wide contraction chunks of the head dim
  static constexpr int KCHT = KCH + (AUG ? 1 : 0);  // plus one chunk of bias one-hots
  static constexpr int DK = KCHT * 32;
  // The ones row needs an extra 16-row block when D is a multiple of 16; at
  // D = 80 that block does not fit the two-waves-per-SIMD register budget.
  static constexpr bool ONES = kOnesRow && !AUG && (D % 16 != 0 || D <= 64);
  static constexpr int CB = ONES ? D / 16 + 1 : (D + 15) / 16;  // 16-row blocks of O^T
  static constexpr int DV = CB * 16;
  static constexpr int KROW = DK + kKPad;  // LDS row strides (elements)
  static constexpr int VROW = DV + v_row_pad(DV);
  static constexpr int RCH = D / 8;          // 16-byte chunks per token row
  static constexpr int NCH = BN * RCH;
  static constexpr int CPT = (NCH + NT - 1) / NT;
  static constexpr int K_ELEMS = BN * KROW;  // per stage
  static constexpr int V_ELEMS = BN * VROW;
  static constexpr size_t KV_BYTES = 2 * (size_t)(K_ELEMS + V_ELEMS) * 2;
  static constexpr int GROW = 132;           // relpos prologue scratch row (floats)
  static constexpr size_t SCRATCH_BYTES = (size_t)NW * 16 * GROW * 4;
  static constexpr size_t BASE_BYTES =
      ((KV_BYTES > SCRATCH_BYTES ? KV_BYTES : SCRATCH_BYTES) + 15) / 16 * 16;
};

// Scratch row (floats) of the augmented prologue: the <= 62 rows of the
// stacked table [Rh; Rw] for one query, padded to keep 16-byte stores aligned.
constexpr int kAugGrow = 68;

// Row length (floats) of the relative-position prologue scratch: every
// stored or needed table row of either axis.
constexpr int relpos_grow(const AttnArgs& a) {
  int g = a.gh > a.gw ? a.gh : a.gw;
  g = g > a.kgh ? g : a.kgh;
  g = g > a.kgw ? g : a.kgw;
  int m = 2 * g - 1;
  m = m > a.rh_rows ? m : a.rh_rows;
  m = m > a.rw_rows ? m : a.rw_rows;
  return (m + 15) / 16 * 16 + 4;
}

// Whether Rh or Rw is stored at another length than the grids need (then
// resized in the kernel).
constexpr bool relpos_resized(const AttnArgs& a) {
  return a.bias_kind == ATTN_BIAS_RELPOS &&
         (a.rh_rows != 2 * (a.gh > a.kgh ? a.gh : a.kgh) - 1 ||
          a.rw_rows != 2 * (a.gw > a.kgw ? a.gw : a.kgw) - 1);
}

constexpr bool needs_kinfo(int bias_kind, bool mask) {
  return bias_kind == ATTN_BIAS_TABLE || bias_kind == ATTN_BIAS_RELPOS || mask;
}

// LDS of the per-key index data and the bias tables of the general form:
// kinfo[Nk], then the head's table column or relh[kgh][bm], relw[kgw][bm].
constexpr size_t dyn_lds_bytes(const AttnArgs& a, int bm) {
  const bool kinfo = a.bias_kind == ATTN_BIAS_TABLE || a.bias_kind == ATTN_BIAS_RELPOS ||
                     a.mask_kind == ATTN_MASK_SHIFT_REGIONS;
  size_t n = kinfo ? ((size_t)a.Nk * 4 + 15) / 16 * 16 : 0;
  if (a.bias_kind == ATTN_BIAS_TABLE) n += (size_t)(2 * a.gh - 1) * (2 * a.gw - 1) * 4;
  if (a.bias_kind == ATTN_BIAS_RELPOS) n += (size_t)(a.kgh + a.kgw) * bm * 4;
  return n;
}

// Image layout: the window-map pixel of every key of the workgroup's unit,
// computed once and read by the K/V tile loads (at the end of the LDS).
constexpr size_t img_key_bytes(const AttnArgs& a) {
  return a.image ? ((size_t)a.Nk * 4 + 15) / 16 * 16 : 0;
}

// Dynamic LDS bytes of one workgroup of the tiled kernel.
template <int D, int NW, int NQB, int RMODE = kRelTables>
constexpr size_t mfma_lds_bytes(const AttnArgs& a) {
  using C = MfmaCfg<D, NW, NQB, RMODE == kRelAug>;
  if (RMODE == kRelRow64) return C::BASE_BYTES + (size_t)a.gh * C::BM * 4 + img_key_bytes(a);
  if (RMODE == kRelAug) {
    const size_t scr = (size_t)NW * 16 * kAugGrow * 4;  // overlays the K/V tiles
    return (C::KV_BYTES > scr ? C::KV_BYTES : scr) + img_key_bytes(a);
  }
  size_t n = C::KV_BYTES + dyn_lds_bytes(a, C::BM);
  // Relative-position prologue scratch: G[16 queries][2g-1 rows] per wave.
  if (a.bias_kind == ATTN_BIAS_RELPOS) n += (size_t)NW * 16 * relpos_grow(a) * 4;
  return n + img_key_bytes(a);
}

// ---------------------------------------------------------------------------
// Window kernels (at most 64 tokens per unit)
// ---------------------------------------------------------------------------
constexpr int kWinWaves = 4;

template <int D>
struct WinCfg {
  static constexpr int NT = kWinWaves * 64;
  static constexpr int KCH = (D + 31) / 32;
  static constexpr int DK = KCH * 32;
  static constexpr int CB = (D + 15) / 16;
  static constexpr int DV = CB * 16;
  static constexpr int KROW = DK + 8;
  static constexpr int VROW = DV + v_row_pad(DV);
  static constexpr int RCH = D / 8;
  static constexpr int NCH = 64 * RCH;               // 16-byte chunks of a 64-token tile
  static constexpr int CPT = (NCH + NT - 1) / NT;    // per thread
  static constexpr size_t KV_BYTES = (size_t)64 * (KROW + VROW) * 2;
};

// fp32 units on v_mfma_f32_16x16x4_f32: D is the head-dim bucket DMAX (the
// call's head dim is at most DMAX; missing columns are zero).  K is stored
// row-major, V transposed (d rows of 64 keys) so that one 16-byte LDS read
// yields the A operands of four consecutive K-steps.
template <int DMAX>
struct WinCfgF32 {
  static constexpr int NT = kWinWaves * 64;
  static constexpr int QC = DMAX / 4;        // K-steps of QK^T; Q floats per lane
  static constexpr int CB = DMAX / 16;       // 16-row blocks of O^T
  static constexpr int KROW = DMAX + 4;      // floats
  static constexpr int VTROW = 64 + 4;       // floats (keys)
  static constexpr size_t KV_BYTES = ((size_t)64 * KROW + (size_t)DMAX * VTROW) * 4;
};

// Entries of the bias table of a window unit: the relative-position table
// (TABLE bias), or a single zero entry when only the region mask is present.
constexpr int win_tab_entries(const AttnArgs& a) {
  return a.bias_kind == ATTN_BIAS_TABLE ? (2 * a.gh - 1) * (2 * a.gw - 1) : 1;
}

// Bias and region mask come from one LDS table lookup per score when the
// bias is a table and/or the mask is the shifted-window region mask.
constexpr bool win_uses_table(const AttnArgs& a) {
  return a.bias_kind == ATTN_BIAS_TABLE || a.mask_kind == ATTN_MASK_SHIFT_REGIONS;
}

constexpr size_t win_lds_bytes(const AttnArgs& a, size_t kv_bytes) {
  size_t n = kv_bytes + 64 * 4;  // per-key index data
  if (win_uses_table(a)) n += (size_t)9 * win_tab_entries(a) * 4;
  return n;
}

// Packed window kernel: HG heads of a window in one workgroup of 4*HG waves
// (one per head and 16-query block).  Each head's K and V tiles have their
// own LDS region; V carries a ones block (column D) so the row sums come
// from the matrix cores.  The table holds HG floats per entry (one per
// head), in 9 region copies when the region mask is on.
template <int D>
struct WinPackCfg {
  static constexpr int NT = kWinWaves * 64;
  static constexpr int KCH = (D + 31) / 32;
  static constexpr int DK = KCH * 32;
  static constexpr int CB = D / 16 + 1;              // O^T blocks, the last holds the ones row
  static constexpr int DV = CB * 16;
  static constexpr int KROW = DK + 8;
  static constexpr int VROW = DV + v_row_pad(DV);
  static constexpr int RCH = D / 8;
  static constexpr int NCH = 64 * RCH;
  static constexpr int CPT = (NCH + NT - 1) / NT;
  static constexpr size_t HEAD_BYTES = (size_t)64 * (KROW + VROW) * 2;
};

// Whether the packed window kernel can run this call: half precision,
// table or no bias, region or no mask.
constexpr bool win_packable(const AttnArgs& a) {
  return a.dtype != ATTN_F32 && (a.bias_kind == ATTN_BIAS_NONE || a.bias_kind == ATTN_BIAS_TABLE) &&
         a.mask_kind != ATTN_MASK_ADDITIVE;
}

constexpr size_t win_pack_lds_bytes(const AttnArgs& a, size_t head_bytes, int hg) {
  size_t n = head_bytes * hg + 64 * 4;
  if (win_uses_table(a)) {
    const int copies = a.mask_kind == ATTN_MASK_SHIFT_REGIONS ? 9 : 1;
    n += (size_t)copies * win_tab_entries(a) * hg * 4;
  }
  return n;
}

// Window backward kernel (attn_bwd_win): Q, K, V and dO tiles of 64 rows
// (head dim padded to the 32-wide contraction), P^T and dS^T in the element
// type (64 keys x 64 queries, rows padded by 8), dS^T in fp32 for the table
// gradient (rows of 65), then the per-key lookup parts and the table.  (A
// pad of 16, which the tiled backward takes, measured 2 % slower here.)
template <int D>
struct WinBwdCfg {
  static constexpr int NT = kWinWaves * 64;
  static constexpr int KCH = (D + 31) / 32;
  static constexpr int DK = KCH * 32;
  static constexpr int CBD = (D + 15) / 16;   // 16-wide blocks of dQ, dK, dV columns
  static constexpr int ROW = DK + 8;
  static constexpr int PROW = 64 + 8;
  static constexpr int FROW = 64 + 1;
  static constexpr int RCH = D / 8;
  static constexpr int NCH = 64 * RCH;
  static constexpr int CPT = (NCH + NT - 1) / NT;
  static constexpr size_t BYTES = (size_t)4 * 64 * ROW * 2 + (size_t)2 * 64 * PROW * 2 +
                                  (size_t)64 * FROW * 4 + 64 * 4;
};

constexpr size_t win_bwd_lds_bytes(const AttnArgs& a, size_t base) {
  return base + (win_uses_table(a) ? (size_t)9 * win_tab_entries(a) * 4 : 0);
}

// ---------------------------------------------------------------------------
// fp32 tiled kernel
// ---------------------------------------------------------------------------
constexpr int kF32Threads = 64;
constexpr int kF32BN = 32;

// ---------------------------------------------------------------------------
// The plan
// ---------------------------------------------------------------------------
enum : int { kKernWin = 0, kKernWinPacked = 1, kKernMfma = 2, kKernF32 = 3 };

struct Plan {
  int kernel;     // kKern*
  int rmode;      // tiled kernel form (kRel*, kTwoTiles)
  int nw;         // waves per workgroup
  int hg;         // heads per workgroup (packed window kernel)
  int bm;         // queries per workgroup (tiled kernels)
  int64_t blocks; // workgroups
  size_t lds;     // LDS bytes per workgroup (dynamic plus static)
};

// Two-tile form: waves per SIMD, and eight-wave workgroups where that target
// is even (so whole workgroups fill each CU).
template <int D>
constexpr int two_tile_wpe() { return D <= 40 ? 4 : (D <= 64 ? 3 : 2); }
template <int D>
constexpr int two_tile_nw() { return two_tile_wpe<D>() % 2 == 0 ? 8 : 4; }

template <int D, int NW>
constexpr size_t mfma_lds_for(const AttnArgs& a, int rmode) {
  switch (rmode) {
    case kRelRow64: return mfma_lds_bytes<D, NW, kNQB, kRelRow64>(a);
    case kRelAug: return mfma_lds_bytes<D, NW, kNQB, kRelAug>(a);
    case kTwoTiles: return mfma_lds_bytes<D, NW, kNQB, kTwoTiles>(a);
    default: return mfma_lds_bytes<D, NW, kNQB, kRelTables>(a);
  }
}

// Half-precision calls with head dim D.
template <int D>
inline Plan plan_half(const AttnArgs& a) {
  Plan p{};
  const bool mask = a.mask_kind != ATTN_MASK_NONE;
  // 8-bit inputs: built for the one-head window form and the tiled forms
  // without relative position.
  if (a.f8 && (a.bias_kind == ATTN_BIAS_RELPOS || a.win_heads > 1)) {
    p.kernel = -1;
    return p;
  }
  // The per-row log-sum-exp output is written by the one-head window form
  // and the tiled forms.
  if (a.lse && a.win_heads > 1) {
    p.kernel = -1;
    return p;
  }
  if (a.bias_kind != ATTN_BIAS_RELPOS && a.Nq <= 64 && a.Nk <= 64) {
    p.nw = kWinWaves;
    // Heads per workgroup: one unless the caller asks for more (one head
    // per workgroup measured fastest for the Swin windows on MI355X).
    p.hg = a.win_heads > 1 ? a.win_heads : 0;
    if (p.hg) {
      if (!win_packable(a) || p.hg > 4 || a.H % p.hg != 0) {
        p.kernel = -1;  // no such form for this call
        return p;
      }
      p.kernel = kKernWinPacked;
      p.nw = kWinWaves * p.hg;
      p.blocks = (int64_t)a.B * (a.H / p.hg);
      p.lds = win_pack_lds_bytes(a, WinPackCfg<D>::HEAD_BYTES, p.hg);
    } else {
      p.kernel = kKernWin;
      p.hg = 1;
      p.blocks = (int64_t)a.B * a.H;
      p.lds = win_lds_bytes(a, WinCfg<D>::KV_BYTES);
    }
    return p;
  }
  if (a.win_heads > 1) {  // heads per workgroup apply to the window path only
    p.kernel = -1;
    return p;
  }
  p.kernel = kKernMfma;
  p.hg = 1;
  p.nw = 4;
  p.rmode = kRelTables;
  // The row and contraction forms read the tables directly: they take equal
  // grids and tables of the needed length; the table form takes the rest.
  const bool same_grid = a.gh == a.kgh && a.gw == a.kgw && !relpos_resized(a);
  if (a.bias_kind == ATTN_BIAS_RELPOS && !mask) {
    // Long key ranges on a 64-wide grid: eight-wave workgroups whose two
    // wave groups alternate matrix and softmax phases (batched layout).
    if (same_grid && a.gw == 64 && a.Nk >= 1024 && a.Nq >= 256 && !a.image) {
      p.rmode = kRelRow64;
      p.nw = 8;
    } else if (same_grid && a.gw == 64) {
      p.rmode = kRelRow64;
    } else if (same_grid && a.gh + a.gw <= 32) {
      p.rmode = kRelAug;
    }
  } else if (a.bias_kind == ATTN_BIAS_NONE && !mask && a.Nk > 64 && a.Nk <= 128) {
    p.rmode = kTwoTiles;
    p.nw = two_tile_nw<D>();
  }
  p.bm = p.nw * kNQB * 16;
  p.blocks = (int64_t)((a.Nq + p.bm - 1) / p.bm) * a.H * a.B;
  p.lds = p.nw == 8 ? mfma_lds_for<D, 8>(a, p.rmode) : mfma_lds_for<D, 4>(a, p.rmode);
  return p;
}

// fp32 calls; DMAX is the register bucket holding the head dim.
template <int DMAX>
inline Plan plan_f32(const AttnArgs& a) {
  Plan p{};
  p.hg = 1;
  if (a.win_heads > 1) {  // the fp32 path has no packed form
    p.kernel = -1;
    return p;
  }
  if (a.bias_kind != ATTN_BIAS_RELPOS && a.Nq <= 64 && a.Nk <= 64) {
    p.kernel = kKernWin;
    p.nw = kWinWaves;
    p.blocks = (int64_t)a.B * a.H;
    p.lds = win_lds_bytes(a, WinCfgF32<DMAX>::KV_BYTES);
    return p;
  }
  p.kernel = kKernF32;
  p.nw = 1;
  p.bm = kF32Threads;
  p.blocks = (int64_t)((a.Nq + kF32Threads - 1) / kF32Threads) * a.H * a.B;
  p.lds = dyn_lds_bytes(a, kF32Threads) + 2 * (size_t)kF32BN * DMAX * 4;
  return p;
}

// The plan of a validated call: ATTN_OK, or ATTN_E_UNSUPPORTED when its
// workgroup needs more LDS than a CU has or the grid is too large.
inline int make_plan(const AttnArgs& a, Plan* p) {
  switch (a.dtype) {
    case ATTN_F32:
      *p = a.D <= 32 ? plan_f32<32>(a) : a.D <= 64 ? plan_f32<64>(a) : plan_f32<128>(a);
      break;
    default:
      switch (a.D) {
        case 32: *p = plan_half<32>(a); break;
        case 40: *p = plan_half<40>(a); break;
        case 64: *p = plan_half<64>(a); break;
        case 80: *p = plan_half<80>(a); break;
        default: return ATTN_E_UNSUPPORTED;
      }
  }
  if (p->kernel < 0 || p->lds > kMaxLds || p->blocks > 0x7fffffff) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
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
// rel_w stay in registers per key slot).
constexpr int kBwdRelNone = 0, kBwdRelGeneral = 1, kBwdRelRow64 = 2;
constexpr int kBwdRelMaxCols = 84;

constexpr int bwd_rel_mode(const AttnArgs& a) {
  return a.bias_kind != ATTN_BIAS_RELPOS ? kBwdRelNone
         : (a.gw == 64 && a.gh <= 64)     ? kBwdRelRow64
                                          : kBwdRelGeneral;
}

// Rows of the stacked table [Rh; Rw] (equal grids, tables of the needed length).
constexpr int bwd_rel_rows(const AttnArgs& a) { return 2 * a.gh - 1 + 2 * a.gw - 1; }

// Workspace of the tiled backward, in floats: the rows' L and D (B*H*Nq
// each), then with the relative position the rel_h / rel_w rows of every
// query ([B*H*Nq][gh + gw], written by the row kernel, read by the column
// kernel) and one partial [Rh; Rw] gradient per row-kernel workgroup
// ([B*H*ceil(Nq/64)][rows][D], summed in a fixed order afterwards).
// Per-workgroup slot of the partial table gradients (floats): the [dRh; dRw]
// part, and in the 64-wide form first the workgroup's dRelH^T and dRelW^T
// ([gh + 64][64] floats, read back after the key loop).
constexpr size_t bwd_part_stride(const AttnArgs& a) {
  const size_t part = (size_t)bwd_rel_rows(a) * (size_t)a.D;
  const size_t drel = bwd_rel_mode(a) == kBwdRelRow64 ? (size_t)(a.gh + 64) * 64 : 0;
  return part > drel ? part : drel;
}
struct BwdWs {
  size_t L, D, rel, part, pstride, total;
};
constexpr BwdWs bwd_ws_layout(const AttnArgs& a) {
  const size_t n = (size_t)a.B * a.H * a.Nq;
  BwdWs w{0, n, 0, 0, 0, 0};
  size_t off = (2 * n + 3) / 4 * 4;
  w.rel = off;
  if (a.bias_kind == ATTN_BIAS_RELPOS) {
    off = (off + n * (size_t)(a.gh + a.gw) + 3) / 4 * 4;
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
// Bytes of the per-lane dRel sums at the end of the relative-position
// region (general grids).
constexpr size_t bwd_rows_acc_bytes(const AttnArgs& a) {
  return bwd_rel_mode(a) == kBwdRelGeneral ? (size_t)256 * ((a.gh + a.gw) | 1) * 4 : 0;
}
template <int D>
constexpr size_t bwd_rows_rel_bytes(const AttnArgs& a) {
  constexpr int ROW = (D + 31) / 32 * 32 + kBwdRowPad;
  const int mode = bwd_rel_mode(a);
  if (mode == kBwdRelNone) return 0;
  const size_t g = (size_t)(a.gh + a.gw);
  size_t rel = mode == kBwdRelGeneral ? 64 * g * 4 : 0;
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
// column from the workspace).
constexpr int bwd_cols_rel_cols(const AttnArgs& a) {
  return bwd_rel_mode(a) == kBwdRelGeneral ? a.gh + a.gw : 0;
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
    p.lds = win_bwd_lds_bytes(a, WinBwdCfg<D>::BYTES);
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
  const size_t cols = (size_t)4 * 64 * ROW * 2 + 4 * 64 * 4 + (size_t)2 * 64 * bwd_cols_rel_cols(a) * 4;
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

#endif  // ATTN_PLAN_H_
