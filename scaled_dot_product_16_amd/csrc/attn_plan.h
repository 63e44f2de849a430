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
  int bm;         // queries per workgroup and tile (tiled kernels)
  int tpw;        // two-tile form, batched layout: query tiles per workgroup
  int64_t blocks; // workgroups
  size_t lds;     // LDS bytes per workgroup (dynamic plus static)
};

// Two-tile form: waves per SIMD, and eight-wave workgroups where that target
// is even (so whole workgroups fill each CU).
template <int D>
constexpr int two_tile_wpe() { return D <= 40 ? 4 : (D <= 64 ? 3 : 2); }
template <int D>
constexpr int two_tile_nw() { return two_tile_wpe<D>() % 2 == 0 ? 8 : 4; }
// Two-tile form in the batched layout: each workgroup keeps the K and V
// tiles of its (batch item, head) in LDS and walks tpw consecutive query
// tiles, the next tile's Q in flight during the current one, so that the
// grid is about one round of resident workgroups (256 CUs of the chip).
// Its output is staged through a region of its own (NW * NQB * 16 * D
// elements) instead of the K/V stages.  Not at d = 64, where that region
// would leave two resident workgroups per CU instead of three.
constexpr int kPersistCUs = 256;
template <int D>
constexpr int two_tile_tpw(const AttnArgs& a, int bm) {
  const int64_t per_unit = (a.Nq + bm - 1) / bm;
  const int64_t total = per_unit * a.H * a.B;
  const int64_t slots = (int64_t)kPersistCUs * (4 * two_tile_wpe<D>() / two_tile_nw<D>());
  int64_t t = (total + slots - 1) / slots;
  if (t > per_unit) t = per_unit;
  return t < 1 ? 1 : (int)t;
}
template <int D>
constexpr size_t two_tile_stage_bytes() { return (size_t)two_tile_nw<D>() * kNQB * 16 * D * 2; }
template <int D>
constexpr bool two_tile_persists() { return D != 64; }

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
  p.tpw = 1;
  p.blocks = (int64_t)((a.Nq + p.bm - 1) / p.bm) * a.H * a.B;
  p.lds = p.nw == 8 ? mfma_lds_for<D, 8>(a, p.rmode) : mfma_lds_for<D, 4>(a, p.rmode);
  if (p.rmode == kTwoTiles && !a.image && two_tile_persists<D>()) {
    p.tpw = two_tile_tpw<D>(a, p.bm);
    const int64_t per_unit = (a.Nq + p.bm - 1) / p.bm;
    p.blocks = (per_unit + p.tpw - 1) / p.tpw * a.H * a.B;
    p.lds = (p.lds + 15) / 16 * 16 + two_tile_stage_bytes<D>();
  }
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

}  // namespace attn

// The backward kernels' geometry and plan.
#include "attn_plan_bwd.h"

#endif  // ATTN_PLAN_H_
