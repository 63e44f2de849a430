// Short-sequence attention (windows of up to 64 tokens) on gfx950.
//
// Swin-style window attention has many small, independent (window, head)
// units: 49 tokens each for 7x7 windows.  One workgroup of four waves owns
// one unit and keeps all of it on chip: wave w holds queries 16w..16w+15 as
// MFMA operands in registers, K and V of the whole unit are staged once in
// LDS (V read back transposed), the 64-key score tile (keys past N start
// from -inf) lives in registers, and the softmax needs no running rescale
// because the whole key range is one tile.  Table bias indices, region
// labels and the image addressing of the window partition and cyclic shift
// (Swin talk, sections 1 and 2) are computed from per-lane token
// coordinates.
#ifndef ATTN_WIN_H_
#define ATTN_WIN_H_

#include <type_traits>

#include "attn_mfma.h"

namespace attn {

// Tile geometry (WinCfg, WinCfgF32, WinPackCfg) and the LDS byte counts are
// in attn_plan.h, shared with the host-side kernel choice.

// Per-unit window placement (image layout and region labels).
struct WinPos {
  int img;     // image index (image layout)
  int y0, x0;  // shifted-image origin of the window
};

__device__ __forceinline__ WinPos win_pos(const AttnArgs& a, int b) {
  WinPos p;
  // Without window geometry nw = nwx = 0 and both divisors are 1: the
  // origin below is then (0, 0).
  p.img = fdiv(b, a.fd_nw);
  const int w = b - p.img * a.nw;
  const int wy = fdiv(w, a.fd_nwx);
  const int wx = w - wy * a.nwx;
  p.y0 = wy * a.win_h;
  p.x0 = wx * a.win_w;
  return p;
}

// Image pixel of window token (ty, tx) inside one (image, head) slice, or
// kPadTok for a padding token.
__device__ __forceinline__ uint32_t win_tok_pix(const AttnArgs& a, const WinPos& p, int ty, int tx) {
  const int pix = image_pixel(a, p.y0, p.x0, ty, tx);
  return pix < 0 ? kPadTok : (uint32_t)pix;
}

__device__ __forceinline__ int win_region(const AttnArgs& a, const WinPos& p, int ty, int tx) {
  const int y = p.y0 + ty, x = p.x0 + tx;
  const int ry = y < a.pimg_h - a.win_h ? 0 : (y < a.pimg_h - a.shift_h ? 1 : 2);
  const int rx = x < a.pimg_w - a.win_w ? 0 : (x < a.pimg_w - a.shift_w ? 1 : 2);
  return 3 * ry + rx;
}

// One workgroup = one (batch item, head) unit of at most 64 tokens; wave w
// owns queries 16w .. 16w+15.  MASKK: ATTN_MASK_NONE / _ADDITIVE /
// _SHIFT_REGIONS.
//
// Table bias and region mask share one LDS lookup per score.  The table of
// n entries is stored 9 times: copy c = 3*(dy+1) + (dx+1) holds the table
// plus the mask value, except copy 4 (dy = dx = 0), where dy and dx are the
// differences of the query's and the key's region labels along each axis
// (in a window they differ by at most one).  The lookup address splits into
// a per-query part and a per-key part:
//   idx(q) - idx(k) + n * c  =  [idx(q) + n*(3*ry_q + rx_q)]
//                              + [4n - idx(k) - n*(3*ry_k + rx_k)],
// with idx(q) = (qh+gh-1)(2gw-1) + qw+gw-1 and idx(k) = kh(2gw-1) + kw, so
// each score costs one add and one LDS read.
//
// E = F32E selects the fp32 form (WinCfgF32): same structure, with
// v_mfma_f32_16x16x4_f32 products and fp32 tiles.
//
// F8: q, k and v are E4M3 codes (half precision only).  They are loaded as
// 8-byte pieces, widened exactly to E in registers and then take the same
// path; the q and k scales ride in a.scale and the v scale is applied with
// the row-sum division.
template <class E, int D, int BIAS, int MASKK, bool F8 = false>
__global__ __launch_bounds__(kWinWaves * 64) void attn_fwd_win(AttnArgs a) {
  constexpr bool F32 = std::is_same<E, F32E>::value;
  static_assert(!(F8 && F32), "8-bit inputs are widened to a half-precision type");
  using C = WinCfg<F32 ? 32 : D>;
  using CF = WinCfgF32<F32 ? D : 32>;
  constexpr int NT = C::NT, KCH = C::KCH, CB = F32 ? CF::CB : C::CB, KROW = C::KROW, VROW = C::VROW,
                RCH = C::RCH, NCH = C::NCH, CPT = C::CPT, DK = C::DK, DV = C::DV;
  constexpr size_t kKvBytes = F32 ? CF::KV_BYTES : C::KV_BYTES;
  constexpr bool kTab = BIAS == ATTN_BIAS_TABLE || MASKK == ATTN_MASK_SHIFT_REGIONS;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* Ks = (uint16_t*)lds;        // [64][KROW]
  uint16_t* Vs = Ks + 64 * KROW;        // [64][VROW]
  float* Kf = (float*)lds;              // fp32: [64][CF::KROW]
  float* Vtf = Kf + 64 * CF::KROW;      // fp32: [DMAX][CF::VTROW], V transposed
  int* kinfo = (int*)(lds + kKvBytes);               // per key: byte offset of its table part
  constexpr int kTabByte = (int)kKvBytes + 64 * 4;   // 9 table copies, log2 units
  float* tbl = (float*)(lds + kTabByte);

  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int H = a.H, N = a.Nq, Nk = a.Nk;
  const int unit = xcd_logical_id(__builtin_amdgcn_workgroup_id_x(), a.n_blocks);
  const int b = fdiv(unit, a.fd_h), h = unit - b * H;

  // Token t < 64 of a window -> (row, column) for a row length n <= 1024: the
  // float quotient (t + 0.5) / n is within 2e-5 of the exact value and at
  // least 0.5 / n away from an integer, so truncation is exact.
  const float inv_ww = __builtin_amdgcn_rcpf((float)(a.win_w > 0 ? a.win_w : 1));
  const float inv_gw = __builtin_amdgcn_rcpf((float)(a.gw > 0 ? a.gw : 1));
  auto div_small = [](int t, float inv) { return (int)(((float)t + 0.5f) * inv); };
  auto split = [&](int t, int& ty, int& tx) {
    ty = div_small(t, inv_ww);
    tx = t - ty * a.win_w;
  };
  const WinPos pos = win_pos(a, b);
  const int bimg = a.image ? pos.img : b;
  // Token t -> its row in the (image, head) slice: t itself (batched
  // layout) or the shifted-image pixel of window token t (image layout).
  auto tok_pix = [&](int t) -> uint32_t {
    if (!a.image) return (uint32_t)t;
    int ty, tx;
    split(t, ty, tx);
    return win_tok_pix(a, pos, ty, tx);
  };
  constexpr int ES = F32 ? 4 : 2;  // element bytes
  constexpr int IES = F8 ? 1 : ES;  // element bytes of q, k, v
  const char* qp = (const char*)a.q + ((int64_t)bimg * a.q_sb + (int64_t)h * a.q_sh) * IES;
  const char* kp = (const char*)a.k + ((int64_t)bimg * a.k_sb + (int64_t)h * a.k_sh) * IES;
  const char* vp = (const char*)a.v + ((int64_t)bimg * a.v_sb + (int64_t)h * a.v_sh) * IES;
  char* op = (char*)a.o + ((int64_t)bimg * a.o_sb + (int64_t)h * a.o_sh) * ES;
  using LdT = std::conditional_t<F8, u32x2, u32x4>;  // one 8-element chunk as loaded

  // Global loads first.  Token rows past N are clamped to the last token, so
  // every load is unconditional; those keys start from -inf below, so their
  // probabilities are exactly zero and their finite values never reach O.
  constexpr int FCH = F32 ? 64 * CF::QC : 1;          // fp32: 16-byte chunks of a tile (QC per row)
  constexpr int FCPT = (FCH + NT - 1) / NT;
  LdT kreg[F32 ? FCPT : CPT], vreg[F32 ? FCPT : CPT];
  if constexpr (F32) {
#pragma unroll
    for (int c = 0; c < FCPT; ++c) {
      const int ch = min(tid + c * NT, FCH - 1);
      const int c4 = (ch % CF::QC) * 4;
      const uint32_t pix0 = tok_pix(min(ch / CF::QC, Nk - 1));
      const uint32_t pix = pix0 == kPadTok ? 0u : pix0;
      const int col = c4 < a.D ? c4 : 0;
      kreg[c] = *(const u32x4*)(kp + (size_t)(pix * (uint32_t)a.k_sn + col) * 4);
      vreg[c] = *(const u32x4*)(vp + (size_t)(pix * (uint32_t)a.v_sn + col) * 4);
      if (c4 >= a.D || pix0 == kPadTok) kreg[c] = vreg[c] = u32x4{0, 0, 0, 0};
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = min(tid + c * NT, NCH - 1);
      const uint32_t pix0 = tok_pix(min(ch / RCH, Nk - 1));
      const uint32_t pix = pix0 == kPadTok ? 0u : pix0;
      const uint32_t col = (uint32_t)((ch % RCH) * 8);
      // Every q, k and v byte is read by exactly one workgroup: streaming
      // (non-temporal) loads, measured faster for the Swin window shapes.
      kreg[c] = __builtin_nontemporal_load((const LdT*)(kp + (size_t)(pix * (uint32_t)a.k_sn + col) * IES));
      vreg[c] = __builtin_nontemporal_load((const LdT*)(vp + (size_t)(pix * (uint32_t)a.v_sn + col) * IES));
      if (pix0 == kPadTok) kreg[c] = vreg[c] = LdT{};  // padding token (code 0 is +0 too)
    }
  }
  const int q_tok = min(wave * 16 + l16, N - 1);
  const uint32_t q_pix0 = tok_pix(q_tok);
  const bool q_pad = q_pix0 == kPadTok;  // padding token: zero query, output not stored
  const uint32_t q_pix = q_pad ? 0u : q_pix0;
  const uint32_t q_off = q_pix * (uint32_t)a.q_sn;
  u32x4 qf[F32 ? CF::QC / 4 : KCH];
  if constexpr (F32) {
    // K-step dc of this lane's group g covers column g*QC + dc.
#pragma unroll
    for (int j = 0; j < CF::QC / 4; ++j) {
      const int d0 = g * CF::QC + 4 * j;
      qf[j] = d0 < a.D && !q_pad ? *(const u32x4*)(qp + (size_t)(q_off + d0) * 4) : u32x4{0, 0, 0, 0};
    }
  } else {
#pragma unroll
    for (int dc = 0; dc < KCH; ++dc) {
      const int d0 = dc * 32 + g * 8;
      if constexpr (F8) {
        // Unconditional load (q_off is a valid row, d0 < D here or clamped),
        // then a select: the load is not waited for inside a branch.
        const bool ok = d0 < D && !q_pad;
        const u32x4 wq = widen_e4m3<E>(__builtin_nontemporal_load((const u32x2*)(qp + q_off + (ok ? d0 : 0))));
        qf[dc] = ok ? wq : u32x4{0, 0, 0, 0};
      } else
        qf[dc] = d0 < D && !q_pad ? __builtin_nontemporal_load((const u32x4*)(qp + (size_t)(q_off + d0) * 2))
                                  : u32x4{0, 0, 0, 0};
    }
  }

  // Only windows on the last window row or column of the shifted image hold
  // more than one region.
  const bool regions = MASKK == ATTN_MASK_SHIFT_REGIONS &&
                       (pos.y0 + a.win_h > a.pimg_h - a.win_h || pos.x0 + a.win_w > a.pimg_w - a.win_w);
  const int n_tab = win_tab_entries(a);
  if constexpr (kTab) {
    const float mv = a.mask_value * kLog2e;
    for (int r = tid; r < n_tab; r += NT) {
      const float t = BIAS == ATTN_BIAS_TABLE ? load_elem<E>(a.table, (int64_t)r * H + h) * kLog2e : 0.f;
      tbl[4 * n_tab + r] = t;
      if (regions) {
#pragma unroll
        for (int c = 0; c < 9; ++c)
          if (c != 4) tbl[c * n_tab + r] = t + mv;
      }
    }
    if (tid < 64) {
      const int j = min(tid, Nk - 1);
      int part = 4 * n_tab;
      if constexpr (BIAS == ATTN_BIAS_TABLE) {
        const int kh = div_small(j, inv_gw), kw = j - kh * a.gw;
        part -= kh * (2 * a.gw - 1) + kw;
      }
      if (regions) {
        int ty, tx;
        split(j, ty, tx);
        part -= n_tab * win_region(a, pos, ty, tx);
      }
      kinfo[tid] = part * 4;
    }
  }
  if constexpr (F32) {
#pragma unroll
    for (int c = 0; c < FCPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < FCH) {
        const int row = ch / CF::QC, c4 = (ch % CF::QC) * 4;
        *(u32x4*)&Kf[row * CF::KROW + c4] = kreg[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) Vtf[(c4 + e) * CF::VTROW + row] = __uint_as_float(vreg[c][e]);
      }
    }
  } else {
    // Padding columns of the tiles are never loaded: zero them.
    if constexpr (DK > D) {
      for (int i = tid; i < 64 * (DK - D); i += NT) Ks[(i / (DK - D)) * KROW + D + i % (DK - D)] = 0;
    }
    if constexpr (DV > D) {
      for (int i = tid; i < 64 * (DV - D); i += NT) Vs[(i / (DV - D)) * VROW + D + i % (DV - D)] = 0;
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < NCH) {
        if constexpr (F8) {
          *(u32x4*)&Ks[(ch / RCH) * KROW + (ch % RCH) * 8] = widen_e4m3<E>(kreg[c]);
          *(u32x4*)&Vs[(ch / RCH) * VROW + (ch % RCH) * 8] = widen_e4m3<E>(vreg[c]);
        } else {
          *(u32x4*)&Ks[(ch / RCH) * KROW + (ch % RCH) * 8] = kreg[c];
          *(u32x4*)&Vs[(ch / RCH) * VROW + (ch % RCH) * 8] = vreg[c];
        }
      }
    }
  }
  __syncthreads();
  if (wave * 16 >= N) return;  // no barrier below this point

  // S^T = K Q^T for the 4 key blocks; keys past Nk (only in a block that
  // reaches past Nk) start from -inf.
  f32x4 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kb * 16 + 16 > Nk) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kb * 16 + g * 4 + r >= Nk) s[kb][r] = -INFINITY;
    }
    if constexpr (F32) {
#pragma unroll
      for (int j = 0; j < CF::QC / 4; ++j) {
        const f32x4 kv = *(const f32x4*)&Kf[(kb * 16 + l16) * CF::KROW + g * CF::QC + 4 * j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], __uint_as_float(qf[j][e]), s[kb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int dc = 0; dc < KCH; ++dc) {
        const u32x4 kf = *(const u32x4*)&Ks[(kb * 16 + l16) * KROW + dc * 32 + g * 8];
        s[kb] = E::mfma(kf, qf[dc], s[kb]);
      }
    }
  }

  // Bias and mask (log2 units): a table lookup (table bias and/or region
  // mask) plus dense additive terms (additive bias and/or mask); a call may
  // have both, e.g. a table bias with an additive mask.
  const float c2 = a.scale * kLog2e;
  constexpr bool kDense = BIAS == ATTN_BIAS_ADDITIVE || MASKK == ATTN_MASK_ADDITIVE;
  auto dense = [&](int kb, int r) -> float {
    const int j = min(kb * 16 + g * 4 + r, Nk - 1);
    float t = 0.f;
    if constexpr (BIAS == ATTN_BIAS_ADDITIVE)
      t = load_elem<E>(a.badd, (int64_t)(b % a.badd_n) * a.badd_s0 + (int64_t)q_tok * a.badd_s1 + j) * kLog2e;
    if constexpr (MASKK == ATTN_MASK_ADDITIVE)
      t += load_elem<E>(a.madd, (int64_t)(b % a.madd_n) * a.madd_s0 + (int64_t)q_tok * a.madd_s1 + j) * kLog2e;
    return t;
  };
  float y[16];
  if constexpr (kTab) {
    int qpart = 0;
    if constexpr (BIAS == ATTN_BIAS_TABLE) {
      const int qh = div_small(q_tok, inv_gw), qw = q_tok - qh * a.gw;
      qpart = (qh + a.gh - 1) * (2 * a.gw - 1) + qw + a.gw - 1;
    }
    if (regions) {
      int ty, tx;
      split(q_tok, ty, tx);
      qpart += n_tab * win_region(a, pos, ty, tx);
    }
    const char* qbase = lds + kTabByte + qpart * 4;
    // This lane's keys are kb*16 + g*4 + r: four consecutive kinfo entries.
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 v = *(const u32x4*)&kinfo[kb * 16 + g * 4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float t = *(const float*)(qbase + (int)v[r]);
        if constexpr (kDense) t += dense(kb, r);
        y[kb * 4 + r] = fmaf(s[kb][r], c2, t);
      }
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[kb * 4 + r] = fmaf(s[kb][r], c2, dense(kb, r));
  }

  // Softmax over the single key tile.
  float mx = fmaxf(fmaxf(y[0], y[1]), y[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, y[i]), y[i + 1]);
  mx = max_across_groups(fmaxf(mx, y[15]));
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    y[i] = __builtin_amdgcn_exp2f(y[i] - mx);
    ps += y[i];
  }
  f32x4 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (F32) {
    // O^T += V^T P^T over K-steps of 4 keys {kb*16 + 4k + r : k = 0..3}:
    // this lane's own probability of key kb*16 + 4g + r is the B operand.
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const f32x4 vt = *(const f32x4*)&Vtf[(cb * 16 + l16) * CF::VTROW + kb * 16 + g * 4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vt[r], y[kb * 4 + r], o[cb], 0, 0, 0);
      }
  } else {
    u32x4 pf[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
      pf[kc] = u32x4{E::pack2(y[kc * 8 + 0], y[kc * 8 + 1]), E::pack2(y[kc * 8 + 2], y[kc * 8 + 3]),
                     E::pack2(y[kc * 8 + 4], y[kc * 8 + 5]), E::pack2(y[kc * 8 + 6], y[kc * 8 + 7])};
    // O^T += V^T P^T with transposing reads of the V tile.
    const int vt_row = g * 4 + (l16 >> 2), vt_col = 4 * (l16 & 3);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint16_t* vptr = Vs + (kc * 32 + vt_row) * VROW + cb * 16 + vt_col;
        const u32x2 lo = lds_read_tr16(vptr);
        const u32x2 hi = lds_read_tr16(vptr + 16 * VROW);
        o[cb] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kc], o[cb]);
      }
  }

  const float tot = sum_across_groups(ps);
  float inv = F32 ? 1.f / tot : __builtin_amdgcn_rcpf(tot);
  if constexpr (F8) inv *= a.v_descale;
  if constexpr (!F32) {
    // Row log-sum-exp (natural log): mx is the row maximum in log2 units.
    if (a.lse && g == 0 && wave * 16 + l16 < N && !q_pad) {
      const int ntok = a.image ? a.img_h * a.img_w : N;
      a.lse[((int64_t)bimg * H + h) * ntok + q_pix] = (mx + __builtin_amdgcn_logf(tot)) * kLn2;
    }
  }
  if (wave * 16 + l16 < N && !q_pad) {
    // Query row wave*16 + l16 is q_tok here, so its pixel is q_pix.
    const uint32_t off = q_pix * (uint32_t)a.o_sn;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c0 = cb * 16 + g * 4;
      if (c0 < (F32 ? a.D : D)) {
        const f32x4 v = o[cb] * inv;
        if constexpr (F32) *(f32x4*)(op + (size_t)(off + c0) * 4) = v;
        // O is written once and never read here: streaming (non-temporal)
        // stores, measured faster for the Swin window shapes.
        else __builtin_nontemporal_store(u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])},
                                         (u32x2*)(op + (size_t)(off + c0) * 2));
      }
    }
  }
}

// Packed short-sequence form: one workgroup owns one window and HG of its
// heads (all heads of a Swin window when HG = H), one wave per (head,
// 16-query block): 4*HG waves.  The work that depends on the window only --
// the per-key table offsets and region labels, and the staging of the bias
// table, which holds HG floats per entry (one per head) -- is done once for
// the HG heads; every wave then runs one head's 16 queries exactly as
// attn_fwd_win runs a unit's, reading its head's bias at an immediate offset.
// On gfx950 the window shapes are bound by the length of each wave's chain
// of load, lookup, softmax and store rather than by instruction issue, so
// the waves stay as short as in the one-unit form (measured: four waves
// that each ran all HG heads were 1.3x slower for Swin-T, whether the heads
// ran one after another or side by side).  V carries a ones block (column D),
// so the row sums come out of the P.V products.
// BIAS: ATTN_BIAS_NONE / _TABLE; MASKK: ATTN_MASK_NONE / _SHIFT_REGIONS.
template <class E, int D, int HG, int BIAS, int MASKK>
__global__ __launch_bounds__(kWinWaves * HG * 64) void attn_fwd_winp(AttnArgs a) {
  using C = WinPackCfg<D>;
  constexpr int NTH = C::NT;                 // threads staging one head's tiles
  constexpr int NT = NTH * HG;               // threads of the workgroup
  constexpr int KCH = C::KCH, CB = C::CB, KROW = C::KROW, VROW = C::VROW, RCH = C::RCH,
                NCH = C::NCH, CPT = C::CPT, DK = C::DK, DV = C::DV;
  constexpr int K_ELEMS = 64 * KROW, HEAD_ELEMS = (int)(C::HEAD_BYTES / 2);
  constexpr bool kTab = BIAS == ATTN_BIAS_TABLE || MASKK == ATTN_MASK_SHIFT_REGIONS;
  constexpr bool kRegions = MASKK == ATTN_MASK_SHIFT_REGIONS;
  // Region copy the lookup lands in when query and key share a region.
  constexpr int kCopy0 = kRegions ? 4 : 0;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* tiles = (uint16_t*)lds;                    // head j: K [64][KROW], V [64][VROW]
  int* kinfo = (int*)(lds + HG * C::HEAD_BYTES);       // per key: byte offset of its table part
  constexpr int kTabByte = HG * (int)C::HEAD_BYTES + 64 * 4;
  float* tbl = (float*)(lds + kTabByte);               // [copy][entry][HG], log2 units

  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = wave >> 2, qb = wave & 3;              // this wave's head and query block
  const int ht = tid - j * NTH;                        // thread index inside its head's group
  const int l16 = lane & 15, g = lane >> 4;
  const int H = a.H, N = a.Nq, Nk = a.Nk;
  const int unit = xcd_logical_id(__builtin_amdgcn_workgroup_id_x(), a.n_blocks);
  const int b = fdiv(unit, a.fd_hgrp), h0 = (unit - b * a.n_hgrp) * HG;

  // Token t < 64 -> (row, column) by a float reciprocal (exact for n <= 1024,
  // as in attn_fwd_win).
  const float inv_ww = __builtin_amdgcn_rcpf((float)(a.win_w > 0 ? a.win_w : 1));
  const float inv_gw = __builtin_amdgcn_rcpf((float)(a.gw > 0 ? a.gw : 1));
  auto div_small = [](int t, float inv) { return (int)(((float)t + 0.5f) * inv); };
  auto split = [&](int t, int& ty, int& tx) {
    ty = div_small(t, inv_ww);
    tx = t - ty * a.win_w;
  };
  const WinPos pos = win_pos(a, b);
  const int bimg = a.image ? pos.img : b;
  auto tok_pix = [&](int t) -> uint32_t {
    if (!a.image) return (uint32_t)t;
    int ty, tx;
    split(t, ty, tx);
    return win_tok_pix(a, pos, ty, tx);
  };
  // Byte bases of this wave's head.
  const int h = h0 + j;
  const char* qp = (const char*)a.q + ((int64_t)bimg * a.q_sb + (int64_t)h * a.q_sh) * 2;
  const char* kp = (const char*)a.k + ((int64_t)bimg * a.k_sb + (int64_t)h * a.k_sh) * 2;
  const char* vp = (const char*)a.v + ((int64_t)bimg * a.v_sb + (int64_t)h * a.v_sh) * 2;
  char* op = (char*)a.o + ((int64_t)bimg * a.o_sb + (int64_t)h * a.o_sh) * 2;

  // Loads first: this thread's K/V chunks of its head (token rows past Nk
  // clamped to the last key, whose scores start from -inf below) and this
  // lane's query fragments.  Every byte is read by one workgroup: streaming
  // (non-temporal) loads.
  u32x4 kreg[CPT], vreg[CPT], qf[KCH];
  bool kpad[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = min(ht + c * NTH, NCH - 1);
    const uint32_t pix0 = tok_pix(min(ch / RCH, Nk - 1));
    kpad[c] = pix0 == kPadTok;
    const uint32_t pix = kpad[c] ? 0u : pix0;
    const uint32_t col = (uint32_t)((ch % RCH) * 8);
    kreg[c] = __builtin_nontemporal_load((const u32x4*)(kp + (pix * (uint32_t)a.k_sn + col) * 2));
    vreg[c] = __builtin_nontemporal_load((const u32x4*)(vp + (pix * (uint32_t)a.v_sn + col) * 2));
  }
  const int q_tok = min(qb * 16 + l16, N - 1);
  const uint32_t q_pix0 = tok_pix(q_tok);
  const bool q_pad = q_pix0 == kPadTok;  // padding token: zero query, output not stored
  const uint32_t q_pix = q_pad ? 0u : q_pix0;
#pragma unroll
  for (int dc = 0; dc < KCH; ++dc) {
    const int d0 = dc * 32 + g * 8;
    qf[dc] = d0 < D && !q_pad
                 ? __builtin_nontemporal_load((const u32x4*)(qp + (size_t)(q_pix * (uint32_t)a.q_sn + d0) * 2))
                 : u32x4{0, 0, 0, 0};
  }

  // Padding columns of the head's tiles (independent of the loads): K
  // columns D..DK are zero; V column D is one (the row-sum column), the
  // rest of its last block zero.
  constexpr int KPC = (DK - D) / 8, VPC = (DV - D) / 8;  // 16-byte chunks per row
  uint16_t* Ks = tiles + j * HEAD_ELEMS;
  uint16_t* Vs = Ks + K_ELEMS;
  for (int i = ht; i < 64 * (KPC + VPC); i += NTH) {
    const int row = i / (KPC + VPC), cc = i - row * (KPC + VPC);
    if (cc < KPC) {
      *(u32x4*)&Ks[row * KROW + D + cc * 8] = u32x4{0, 0, 0, 0};
    } else {
      const int vc = cc - KPC;
      *(u32x4*)&Vs[row * VROW + D + vc * 8] = u32x4{vc == 0 ? (uint32_t)E::one_bits() : 0u, 0, 0, 0};
    }
  }

  // Table (HG heads per entry) and per-key parts of the lookup address.
  const bool regions = kRegions &&
                       (pos.y0 + a.win_h > a.pimg_h - a.win_h || pos.x0 + a.win_w > a.pimg_w - a.win_w);
  const int n_tab = win_tab_entries(a);
  if constexpr (kTab) {
    const float mv = a.mask_value * kLog2e;
    for (int e = tid; e < n_tab * HG; e += NT) {
      const int r = e / HG, jj = e - r * HG;
      const float t = BIAS == ATTN_BIAS_TABLE ? load_elem<E>(a.table, (int64_t)r * H + h0 + jj) * kLog2e : 0.f;
      tbl[kCopy0 * n_tab * HG + e] = t;
      if (regions) {
#pragma unroll
        for (int c = 0; c < 9; ++c)
          if (c != 4) tbl[c * n_tab * HG + e] = t + mv;
      }
    }
    if (tid < 64) {
      const int kk = min(tid, Nk - 1);
      int part = kCopy0 * n_tab;
      if constexpr (BIAS == ATTN_BIAS_TABLE) {
        const int kh = div_small(kk, inv_gw), kw = kk - kh * a.gw;
        part -= kh * (2 * a.gw - 1) + kw;
      }
      if (regions) {
        int ty, tx;
        split(kk, ty, tx);
        part -= n_tab * win_region(a, pos, ty, tx);
      }
      kinfo[tid] = part * HG * 4;
    }
  }

#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = ht + c * NTH;
    if (ch < NCH) {
      *(u32x4*)&Ks[(ch / RCH) * KROW + (ch % RCH) * 8] = kpad[c] ? u32x4{0, 0, 0, 0} : kreg[c];
      *(u32x4*)&Vs[(ch / RCH) * VROW + (ch % RCH) * 8] = kpad[c] ? u32x4{0, 0, 0, 0} : vreg[c];
    }
  }
  __syncthreads();
  if (qb * 16 >= N) return;  // no barrier below this point

  // S^T = K Q^T; keys past Nk start from -inf.
  f32x4 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kb * 16 + 16 > Nk) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kb * 16 + g * 4 + r >= Nk) s[kb][r] = -INFINITY;
    }
#pragma unroll
    for (int dc = 0; dc < KCH; ++dc) {
      const u32x4 kf = *(const u32x4*)&Ks[(kb * 16 + l16) * KROW + dc * 32 + g * 8];
      s[kb] = E::mfma(kf, qf[dc], s[kb]);
    }
  }
  // Bias and mask (log2 units): one table read per score, this wave's head
  // at offset 4*j bytes of the entry.
  const float c2 = a.scale * kLog2e;
  float y[16];
  if constexpr (kTab) {
    int qpart = 0;
    if constexpr (BIAS == ATTN_BIAS_TABLE) {
      const int qh = div_small(q_tok, inv_gw), qw = q_tok - qh * a.gw;
      qpart = (qh + a.gh - 1) * (2 * a.gw - 1) + qw + a.gw - 1;
    }
    if (regions) {
      int ty, tx;
      split(q_tok, ty, tx);
      qpart += n_tab * win_region(a, pos, ty, tx);
    }
    const char* qbase = lds + kTabByte + qpart * HG * 4 + 4 * j;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 v = *(const u32x4*)&kinfo[kb * 16 + g * 4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[kb * 4 + r] = fmaf(s[kb][r], c2, *(const float*)(qbase + (int)v[r]));
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[kb * 4 + r] = s[kb][r] * c2;
  }
  float mx = fmaxf(fmaxf(y[0], y[1]), y[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, y[i]), y[i + 1]);
  mx = max_across_groups(fmaxf(mx, y[15]));
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = __builtin_amdgcn_exp2f(y[i] - mx);
  u32x4 pf[2];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
    pf[kc] = u32x4{E::pack2(y[kc * 8 + 0], y[kc * 8 + 1]), E::pack2(y[kc * 8 + 2], y[kc * 8 + 3]),
                   E::pack2(y[kc * 8 + 4], y[kc * 8 + 5]), E::pack2(y[kc * 8 + 6], y[kc * 8 + 7])};
  // O^T += V^T P^T with transposing reads of the V tile; block CB-1 holds
  // the row sums (the ones column of V).
  const int vt_row = g * 4 + (l16 >> 2), vt_col = 4 * (l16 & 3);
  f32x4 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const uint16_t* vptr = Vs + (kc * 32 + vt_row) * VROW + cb * 16 + vt_col;
      const u32x2 lo = lds_read_tr16(vptr);
      const u32x2 hi = lds_read_tr16(vptr + 16 * VROW);
      o[cb] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kc], o[cb]);
    }
  constexpr int LB = D / 16, LG = (D % 16) / 4, LR = D % 4;  // row-sum element of O^T
  const float inv = __builtin_amdgcn_rcpf(__shfl(o[LB][LR], LG * 16 + l16));
  if (qb * 16 + l16 < N && !q_pad) {
    const uint32_t o_off = q_pix * (uint32_t)a.o_sn;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c0 = cb * 16 + g * 4;
      if (c0 < D) {
        const f32x4 v = o[cb] * inv;
        __builtin_nontemporal_store(u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])},
                                    (u32x2*)(op + (size_t)(o_off + c0) * 2));
      }
    }
  }
}

}  // namespace attn

#endif  // ATTN_WIN_H_
