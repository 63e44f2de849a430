// Backward pass of window attention (at most 64 queries and keys per unit)
// on gfx950: dQ, dK, dV and the gradient of the relative-position bias
// table, for the shifted-window attention the Swin talk trains with a fused
// window op (section 2).  The chain rule of O = softmax(scale*QK^T + B + M) V
// per (window, head):
//   P = softmax(S),  dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(P*dP)),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
//   d_table[r, h] = sum of dS over the pairs of head h that read row r.
// A window is one tile, so P is recomputed exactly (no statistics from the
// forward are needed).  One workgroup of four waves owns one unit; Q, K, V
// and dO are staged in LDS, wave w owns queries 16w..16w+15 for S^T = K Q^T
// and dP^T = V dO^T and keys 16w..16w+15 for dK and dV.  The products run on
// v_mfma_f32_16x16x32 with the layouts of the forward kernel: the transposed
// operands (K^T, Q^T, dO^T) come from transposing LDS reads, dS and P are
// rounded to the element type as MFMA operands.  The table gradient is
// summed per unit in a fixed order (one thread per table row, over the
// unit's pairs with that offset) into a workspace, and a second kernel adds
// the units of each head in order: no atomics, bitwise-deterministic.
#ifndef ATTN_BWD_H_
#define ATTN_BWD_H_

#include "attn_win.h"

namespace attn {

template <class E, int D, int BIAS, int MASKK>
__global__ __launch_bounds__(kWinWaves * 64) void attn_bwd_win(AttnBwdArgs ba) {
  using C = WinBwdCfg<D>;
  constexpr int NT = C::NT, KCH = C::KCH, DK = C::DK, CBD = C::CBD, ROW = C::ROW, PROW = C::PROW,
                RCH = C::RCH, NCH = C::NCH, CPT = C::CPT;
  constexpr int TILE = 64 * ROW;
  constexpr bool kTab = BIAS == ATTN_BIAS_TABLE || MASKK == ATTN_MASK_SHIFT_REGIONS;
  const AttnArgs& a = ba.a;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* Ks = (uint16_t*)lds;          // [64][ROW] each: K, V, Q, dO
  uint16_t* Vs = Ks + TILE;
  uint16_t* Qs = Vs + TILE;
  uint16_t* Os = Qs + TILE;               // dO
  uint16_t* Pt = Os + TILE;               // [64 keys][PROW] P^T, element type
  uint16_t* St = Pt + 64 * PROW;          // [64 keys][PROW] dS^T, element type
  int* kinfo = (int*)(St + 64 * PROW);
  float* tbl = (float*)(kinfo + 64);      // 9 table copies, log2 units
  // dS^T in fp32 for the table gradient, [Nk][Nq + 1], written once the K
  // and V tiles are dead: in their space when it fits, else after the table.
  float* Sf = win_bwd_sf_in_kv<D>(a) ? (float*)lds
                                     : (float*)(lds + C::BYTES + (win_uses_table(a) ? 9 * win_tab_entries(a) * 4 : 0));

  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int H = a.H, N = a.Nq, Nk = a.Nk;
  const int unit = xcd_logical_id(__builtin_amdgcn_workgroup_id_x(), a.n_blocks);
  const int b = fdiv(unit, a.fd_h), h = unit - b * H;

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
  auto base = [&](const void* p, int64_t sb, int64_t sh) {
    return (const char*)p + ((int64_t)bimg * sb + (int64_t)h * sh) * 2;
  };
  const char* qp = base(a.q, a.q_sb, a.q_sh);
  const char* kp = base(a.k, a.k_sb, a.k_sh);
  const char* vp = base(a.v, a.v_sb, a.v_sh);
  const char* op = base(a.o, a.o_sb, a.o_sh);  // dO

  // Tiles: token rows past Nq (q, dO) or Nk (k, v) are clamped to the last
  // row, padding tokens of the image layout read as zero.
  u32x4 reg[4][CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = min(tid + c * NT, NCH - 1);
    const int row = ch / RCH;
    const uint32_t col = (uint32_t)((ch % RCH) * 8);
    const uint32_t kpix0 = tok_pix(min(row, Nk - 1)), qpix0 = tok_pix(min(row, N - 1));
    const uint32_t kpix = kpix0 == kPadTok ? 0u : kpix0, qpix = qpix0 == kPadTok ? 0u : qpix0;
    reg[0][c] = *(const u32x4*)(kp + (size_t)(kpix * (uint32_t)a.k_sn + col) * 2);
    reg[1][c] = *(const u32x4*)(vp + (size_t)(kpix * (uint32_t)a.v_sn + col) * 2);
    reg[2][c] = *(const u32x4*)(qp + (size_t)(qpix * (uint32_t)a.q_sn + col) * 2);
    reg[3][c] = *(const u32x4*)(op + (size_t)(qpix * (uint32_t)a.o_sn + col) * 2);
    if (kpix0 == kPadTok) reg[0][c] = reg[1][c] = u32x4{0, 0, 0, 0};
    if (qpix0 == kPadTok) reg[2][c] = reg[3][c] = u32x4{0, 0, 0, 0};
  }

  // Table (with its region copies) and per-key lookup parts, as in the
  // forward window kernel.
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
  // Head-dim padding columns D..DK of the four tiles are zero.
  if constexpr (DK > D) {
    for (int i = tid; i < 4 * 64 * (DK - D); i += NT) {
      const int t = i / (64 * (DK - D)), r = i - t * 64 * (DK - D);
      Ks[t * TILE + (r / (DK - D)) * ROW + D + r % (DK - D)] = 0;
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT;
    if (ch < NCH) {
#pragma unroll
      for (int t = 0; t < 4; ++t) *(u32x4*)&Ks[t * TILE + (ch / RCH) * ROW + (ch % RCH) * 8] = reg[t][c];
    }
  }
  __syncthreads();

  // ---- Per query block: P, dP, dS; dQ -------------------------------------
  const int qrow = wave * 16 + l16;
  const bool qvalid = qrow < N;
  const int q_tok = min(qrow, N - 1);
  u32x4 qf[KCH], df[KCH];
#pragma unroll
  for (int dc = 0; dc < KCH; ++dc) {
    qf[dc] = *(const u32x4*)&Qs[qrow * ROW + dc * 32 + g * 8];
    df[dc] = *(const u32x4*)&Os[qrow * ROW + dc * 32 + g * 8];
  }
  f32x4 s[4], dp[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    dp[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kb * 16 + 16 > Nk) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kb * 16 + g * 4 + r >= Nk) s[kb][r] = -INFINITY;
    }
#pragma unroll
    for (int dc = 0; dc < KCH; ++dc) {
      const u32x4 kf = *(const u32x4*)&Ks[(kb * 16 + l16) * ROW + dc * 32 + g * 8];
      const u32x4 vf = *(const u32x4*)&Vs[(kb * 16 + l16) * ROW + dc * 32 + g * 8];
      s[kb] = E::mfma(kf, qf[dc], s[kb]);
      dp[kb] = E::mfma(vf, df[dc], dp[kb]);
    }
  }
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
  float p[16];
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
    const char* qbase = (const char*)tbl + qpart * 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 v = *(const u32x4*)&kinfo[kb * 16 + g * 4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float t = *(const float*)(qbase + (int)v[r]);
        if constexpr (kDense) t += dense(kb, r);
        p[kb * 4 + r] = fmaf(s[kb][r], c2, t);
      }
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[kb * 4 + r] = fmaf(s[kb][r], c2, dense(kb, r));
  }
  // Exact softmax of the row (the whole key range is this tile).
  float mx = fmaxf(fmaxf(p[0], p[1]), p[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, p[i]), p[i + 1]);
  mx = max_across_groups(fmaxf(mx, p[15]));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p[i] = __builtin_amdgcn_exp2f(p[i] - mx);
    sum += p[i];
  }
  const float inv = 1.f / sum_across_groups(sum);
  // Rows past Nq take no part in dK and dV: their P and dS are zero.
  float pd = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p[i] = qvalid ? p[i] * inv : 0.f;
    pd = fmaf(p[i], dp[i >> 2][i & 3], pd);
  }
  const float dsum = sum_across_groups(pd);  // sum_j P_ij dP_ij
  float ds[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) ds[i] = p[i] * (dp[i >> 2][i & 3] - dsum);
  // P^T and dS^T of this query column into LDS (keys kb*16 + g*4 + r).
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kb * 16 + g * 4 + r;
      const uint32_t pp = E::pack2(p[kb * 4 + r], ds[kb * 4 + r]);
      Pt[key * PROW + qrow] = (uint16_t)(pp & 0xffff);
      St[key * PROW + qrow] = (uint16_t)(pp >> 16);
    }
  // dQ^T = K^T dS^T: dS^T packed as the B operand (the forward's P layout),
  // K^T from transposing reads of the K tile.
  const int vt_row = g * 4 + (l16 >> 2), vt_col = 4 * (l16 & 3);
  {
    u32x4 sf[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
      sf[kc] = u32x4{E::pack2(ds[kc * 8 + 0], ds[kc * 8 + 1]), E::pack2(ds[kc * 8 + 2], ds[kc * 8 + 3]),
                     E::pack2(ds[kc * 8 + 4], ds[kc * 8 + 5]), E::pack2(ds[kc * 8 + 6], ds[kc * 8 + 7])};
    f32x4 acc[CBD];
#pragma unroll
    for (int cb = 0; cb < CBD; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int cb = 0; cb < CBD; ++cb) {
        const uint16_t* ptr = Ks + (kc * 32 + vt_row) * ROW + cb * 16 + vt_col;
        const u32x2 lo = lds_read_tr16(ptr);
        const u32x2 hi = lds_read_tr16(ptr + 16 * ROW);
        acc[cb] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, sf[kc], acc[cb]);
      }
    const uint32_t qpix = tok_pix(q_tok);
    if (qvalid && qpix != kPadTok) {
      char* dq = (char*)ba.dq + ((int64_t)bimg * ba.dq_sb + (int64_t)h * ba.dq_sh) * 2;
#pragma unroll
      for (int cb = 0; cb < CBD; ++cb) {
        const int c0 = cb * 16 + g * 4;
        if (c0 < D) {
          const f32x4 v = acc[cb] * a.scale;
          *(u32x2*)(dq + (size_t)(qpix * (uint32_t)ba.dq_sn + c0) * 2) =
              u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
        }
      }
    }
  }
  __syncthreads();  // P^T, dS^T complete; the K and V tiles are dead
  const int fs = N + 1;  // row stride of the fp32 dS^T
  if constexpr (BIAS == ATTN_BIAS_TABLE) {
    if (qvalid) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb * 16 + g * 4 + r;
          if (key < Nk) Sf[key * fs + qrow] = ds[kb * 4 + r];
        }
    }
  }

  // ---- Per key block: dK = scale * dS^T Q, dV = P^T dO ----------------------
  // Keys 16w .. 16w+15 are the column block; the contraction runs over the
  // 64 query rows in two chunks, Q^T and dO^T from transposing reads, the B
  // operand from rows of dS^T / P^T in the forward's key-permuted order.
  const int krow = wave * 16 + l16;
  if (wave * 16 < Nk) {
    f32x4 dk[CBD], dv[CBD];
#pragma unroll
    for (int cb = 0; cb < CBD; ++cb) dk[cb] = dv[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x2 s0 = *(const u32x2*)&St[krow * PROW + kc * 32 + g * 4];
      const u32x2 s1 = *(const u32x2*)&St[krow * PROW + kc * 32 + 16 + g * 4];
      const u32x2 p0 = *(const u32x2*)&Pt[krow * PROW + kc * 32 + g * 4];
      const u32x2 p1 = *(const u32x2*)&Pt[krow * PROW + kc * 32 + 16 + g * 4];
      const u32x4 sb = {s0[0], s0[1], s1[0], s1[1]}, pb = {p0[0], p0[1], p1[0], p1[1]};
#pragma unroll
      for (int cb = 0; cb < CBD; ++cb) {
        const uint16_t* qptr = Qs + (kc * 32 + vt_row) * ROW + cb * 16 + vt_col;
        const uint16_t* optr = Os + (kc * 32 + vt_row) * ROW + cb * 16 + vt_col;
        const u32x2 ql = lds_read_tr16(qptr), qh = lds_read_tr16(qptr + 16 * ROW);
        const u32x2 ol = lds_read_tr16(optr), oh = lds_read_tr16(optr + 16 * ROW);
        dk[cb] = E::mfma(u32x4{ql[0], ql[1], qh[0], qh[1]}, sb, dk[cb]);
        dv[cb] = E::mfma(u32x4{ol[0], ol[1], oh[0], oh[1]}, pb, dv[cb]);
      }
    }
    const uint32_t kpix = krow < Nk ? tok_pix(krow) : kPadTok;
    if (kpix != kPadTok) {
      char* dkp = (char*)ba.dk + ((int64_t)bimg * ba.dk_sb + (int64_t)h * ba.dk_sh) * 2;
      char* dvp = (char*)ba.dv + ((int64_t)bimg * ba.dv_sb + (int64_t)h * ba.dv_sh) * 2;
#pragma unroll
      for (int cb = 0; cb < CBD; ++cb) {
        const int c0 = cb * 16 + g * 4;
        if (c0 < D) {
          const f32x4 k4 = dk[cb] * a.scale, v4 = dv[cb];
          *(u32x2*)(dkp + (size_t)(kpix * (uint32_t)ba.dk_sn + c0) * 2) =
              u32x2{E::pack2(k4[0], k4[1]), E::pack2(k4[2], k4[3])};
          *(u32x2*)(dvp + (size_t)(kpix * (uint32_t)ba.dv_sn + c0) * 2) =
              u32x2{E::pack2(v4[0], v4[1]), E::pack2(v4[2], v4[3])};
        }
      }
    }
  }

  // ---- Table gradient of this unit --------------------------------------
  // Row r of the table holds offset (oh, ow) = query - key; its gradient is
  // the sum of dS over the unit's pairs with that offset.  Two fixed-order
  // stages (deterministic): M[qh][kh][ow], the sum over qw - kw = ow of the
  // (query row qh, key row kh) block, for every (qh, kh, ow); then row r,
  // the sum of M[qh][qh - oh][ow] over qh in order.
  if constexpr (BIAS == ATTN_BIAS_TABLE) {
    __syncthreads();  // the fp32 dS^T is complete; Q, dO, P^T and dS^T are dead
    const int gh = a.gh, gw = a.gw, tw = 2 * gw - 1;
    float* Mg = (float*)Pt;  // [gh][gh][tw] floats (at most 4096) in the P^T / dS^T space
    const float inv_tw = __builtin_amdgcn_rcpf((float)tw), inv_gh = __builtin_amdgcn_rcpf((float)gh);
    for (int t = tid; t < gh * gh * tw; t += NT) {
      const int blk = div_small(t, inv_tw), owi = t - blk * tw;
      const int qh = div_small(blk, inv_gh), kh = blk - qh * gh, ow = owi - (gw - 1);
      // Query (qh, qw), key (kh, qw - ow): Sf[(kh*gw + qw - ow) * fs + qh*gw + qw].
      const int base = (kh * gw - ow) * fs + qh * gw;
      float acc = 0.f;
      for (int qw = max(0, ow); qw < min(gw, gw + ow); ++qw) acc += Sf[base + qw * (fs + 1)];
      Mg[t] = acc;
    }
    __syncthreads();
    for (int r = tid; r < n_tab; r += NT) {
      const int ohi = div_small(r, inv_tw), owi = r - ohi * tw, oh = ohi - (gh - 1);
      float acc = 0.f;
      for (int qh = max(0, oh); qh < min(gh, gh + oh); ++qh) acc += Mg[(qh * gh + qh - oh) * tw + owi];
      ba.ws[((int64_t)h * n_tab + r) * a.B + b] = acc;  // [H][n_tab][B]: windows contiguous
    }
  }
}

// d_table[r, h] = sum over the batch items b (windows) of the per-unit
// partial sums ws[h][r][b].  One wave per (row, head), four per workgroup:
// lane l adds windows l, l + 64, ... in order, with the loads of 8 windows
// issued before they are added, then a fixed butterfly across the wave
// (shuffles, no barrier) adds the 64 lane sums; lane 0 holds the same sum
// every run (deterministic).  (A template only so that every compiled
// instance may carry its copy.)
template <int kUnused>
__global__ __launch_bounds__(256) void attn_bwd_table_reduce(const float* ws, float* dtable, int B,
                                                             int H, int n_tab) {
  const int lane = __builtin_amdgcn_workitem_id_x() & 63;
  const int i = __builtin_amdgcn_workgroup_id_x() * 4 + (__builtin_amdgcn_workitem_id_x() >> 6);  // r * H + h
  if (i >= n_tab * H) return;  // whole waves
  const int r = i / H, h = i - r * H;
  const float* src = ws + ((int64_t)h * n_tab + r) * B;
  float acc = 0.f;
  int b = lane;
  for (; b + 7 * 64 < B; b += 8 * 64) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[b + j * 64];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += v[j];
  }
  for (; b < B; b += 64) acc += src[b];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) dtable[i] = acc;
}

// ---------------------------------------------------------------------------
// Backward pass of long sequences (no bias, no mask, batched layout): two
// kernels, no atomics.
//
// Row kernel (attn_bwd_rows): one workgroup of four waves owns 64 queries of
// one (batch item, head), Q and dO rows in registers, and streams the K/V
// tiles twice: (1) with S = QK^T and dP = dO V^T, the row log-sum-exp L
// (base 2) of the scaled logits and D = sum_j P_ij dP_ij, both kept online
// against a running row maximum (D = [sum_j 2^(s_ij - m) dP_ij] /
// [sum_j 2^(s_ij - m)], rescaled when m grows); (2) dS = P (dP - D) with
// P = 2^(s - L) and dQ = scale * dS K.  L and D go to the workspace.
// Column kernel (attn_bwd_cols): one workgroup owns 64 keys, K and V rows in
// registers, and streams Q, dO (and L, D) tiles: S = Q K^T, P, dP = dO V^T,
// dS; dV = P^T dO and dK = scale * dS^T Q accumulate over all queries.
// Both use the forward's MFMA layouts (transposed operands from transposing
// LDS reads, probabilities packed as B operands).  The streamed tiles are
// software-pipelined: the next tile's global loads are issued into registers
// before the current tile's products and written to the other of two LDS
// stages after them, with one barrier per tile.
// ---------------------------------------------------------------------------

template <int D>
struct BwdTileCfg {
  static constexpr int NT = 256;
  static constexpr int KCH = (D + 31) / 32;
  static constexpr int DK = KCH * 32;
  static constexpr int CBD = (D + 15) / 16;
  static constexpr int ROW = DK + kBwdRowPad;
  static constexpr int RCH = D / 8;
  static constexpr int NCH = 64 * RCH;
  static constexpr int CPT = (NCH + NT - 1) / NT;
  static constexpr int TILE = 64 * ROW;  // elements of one staged tile
};

// Wait for every vector-memory load this wave has issued (s_waitcnt with
// vmcnt 0, expcnt and lgkmcnt left at their maxima).  Placed before a key
// loop whose operands include fragments loaded in the prologue: the
// compiler's wait analysis cannot see at the loop head that those loads are
// done, and would otherwise wait in every iteration for the next tile's
// prefetch as well, taking the overlap away.
__device__ __forceinline__ void wait_all_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The CPT 16-byte chunks this thread moves of rows [r0, r0 + 64) of a [N, D]
// slice (rows clamped to N-1): global -> registers, registers -> LDS tile.
template <int D>
__device__ __forceinline__ void load_rows_regs(u32x4* reg, const uint16_t* src, int64_t sn, int r0, int n,
                                               int tid) {
  using C = BwdTileCfg<D>;
#pragma unroll
  for (int c = 0; c < C::CPT; ++c) {
    const int ch = min(tid + c * C::NT, C::NCH - 1);
    const int row = ch / C::RCH, col = (ch % C::RCH) * 8;
    reg[c] = *(const u32x4*)(src + (int64_t)min(r0 + row, n - 1) * sn + col);
  }
}

// Byte offsets, from a tile's first row, of the CPT 16-byte chunks this
// thread moves of a 64-row tile with row stride sn (elements).  Offsets that
// do not fit 32 bits, and chunks past the tile, point past every buffer
// range (they read zero).
template <int D>
__device__ __forceinline__ void tile_chunk_offsets(uint32_t* off, int64_t sn, int tid) {
  using C = BwdTileCfg<D>;
#pragma unroll
  for (int c = 0; c < C::CPT; ++c) {
    const int ch = tid + c * C::NT;
    const int64_t o = 2 * ((int64_t)(ch / C::RCH) * sn + (ch % C::RCH) * 8);
    off[c] = ch < C::NCH && o < 0xFFFFFFF0ll ? (uint32_t)o : 0xFFFFFFF0u;
  }
}

// Rows [r0, r0 + 64) of an [n, D] slice at src (r0 < n) into registers
// through a raw buffer resource that ends with row n-1: rows past the slice
// read as zero.  The resource base is uniform, so the per-tile address work
// is scalar; the per-chunk offsets come from tile_chunk_offsets.
template <int D>
__device__ __forceinline__ void load_tile_regs(u32x4* reg, const uint16_t* src, int64_t sn, int r0, int n,
                                               const uint32_t* off) {
  using C = BwdTileCfg<D>;
  const int64_t span = 2 * ((int64_t)(n - 1 - r0) * sn + D);
  const auto rs = buffer_rsrc(src + (int64_t)r0 * sn, span < 0xFFFFFFF0ll ? (uint32_t)span : 0xFFFFFFF0u);
#pragma unroll
  for (int c = 0; c < C::CPT; ++c) {
    reg[c] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[c], 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void store_rows_regs(uint16_t* tile, const u32x4* reg, int tid) {
  using C = BwdTileCfg<D>;
#pragma unroll
  for (int c = 0; c < C::CPT; ++c) {
    const int ch = tid + c * C::NT;
    if (ch < C::NCH) *(u32x4*)&tile[(ch / C::RCH) * C::ROW + (ch % C::RCH) * 8] = reg[c];
  }
}

// Zero the head-dim padding columns [D, DK) of `ntile` staged tiles.
template <int D>
__device__ __forceinline__ void zero_pad_cols(uint16_t* tiles, int ntile, int tid) {
  using C = BwdTileCfg<D>;
  if constexpr (C::DK > D) {
    constexpr int P = C::DK - D;
    for (int i = tid; i < ntile * 64 * P; i += C::NT) {
      const int t = i / (64 * P), r = i - t * 64 * P;
      tiles[t * C::TILE + (r / P) * C::ROW + D + r % P] = 0;
    }
  }
}

// RP: relative-position form (kBwdRelNone / kBwdRelGeneral / kBwdRelRow64).
// With the relative position (equal gh x gw grids, tables of 2g-1 rows) the
// bias of query i and key j = (kh, kw) is rel_h[i][kh] + rel_w[i][kw],
// rel_h[i][kh] = q_i . Rh[qh_i - kh + gh - 1] (rel_w likewise); the row
// kernel computes these rows for its 64 queries (and stores them for the
// column kernel), adds the bias to every score, and in its second pass also
// gathers dRelH[i][kh] = sum over kw of dS and dRelW[i][kw] = sum over kh.
// After the key loop it builds the banded coefficient matrix
//   A[r][i] = dRelH[i][qh_i + gh - 1 - r]  (Rh rows r; Rw rows likewise),
// adds the bias path to dQ,
//   dQ_i += sum_kh dRelH[i][kh] Rh[..] + sum_kw dRelW[i][kw] Rw[..] = sum_r A[r][i] [Rh; Rw][r],
// and writes this workgroup's part of the table gradients,
//   [dRh; dRw][r][c] = sum_i A[r][i] Q[i][c],
// both as small MFMA products over A.
//
// QB: 16-query blocks per wave (a workgroup covers 64 QB queries).  With
// QB = 2 every fragment read from the staged K / V tiles feeds two
// products (no relative position).
template <class E, int D, int RP = kBwdRelNone, int QB = 1>
__global__ __launch_bounds__(256) void attn_bwd_rows(AttnBwdArgs ba) {
  static_assert(QB == 1 || (QB == 2 && RP == kBwdRelNone), "two query blocks per wave: no relative position");
  using C = BwdTileCfg<D>;
  constexpr int KCH = C::KCH, CBD = C::CBD, ROW = C::ROW, TILE = C::TILE;
  const AttnArgs& a = ba.a;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* Ks = (uint16_t*)lds;  // [2][64][ROW]
  uint16_t* Vs = Ks + 2 * TILE;   // [2][64][ROW]
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int bid = xcd_logical_id(__builtin_amdgcn_workgroup_id_x(), a.n_blocks);
  const int qt_div = fdiv(bid, a.fd_qt);
  const int qt = bid - qt_div * a.n_qtiles;
  const int b = fdiv(qt_div, a.fd_h), h = qt_div - b * a.H;
  const int Nq = a.Nq, Nk = a.Nk;
  const int qloc = wave * 16 * QB + l16;  // query of block j: qloc + 16 j
  const int qrow = qt * 64 * QB + qloc;
  const int qi = min(qrow, Nq - 1);
  const uint16_t* qp = (const uint16_t*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const uint16_t* kp = (const uint16_t*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const uint16_t* vp = (const uint16_t*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  const uint16_t* op = (const uint16_t*)a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;  // dO
  const int ntiles = (Nk + 63) / 64;
  u32x4 kreg[C::CPT], vreg[C::CPT];
  uint32_t koff[C::CPT], voff[C::CPT];
  tile_chunk_offsets<D>(koff, a.k_sn, tid);
  tile_chunk_offsets<D>(voff, a.v_sn, tid);
  load_tile_regs<D>(kreg, kp, a.k_sn, 0, Nk, koff);
  load_tile_regs<D>(vreg, vp, a.v_sn, 0, Nk, voff);
  u32x4 qf[QB][KCH], df[QB][KCH];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int qj = min(qrow + 16 * j, Nq - 1);
#pragma unroll
    for (int dc = 0; dc < KCH; ++dc) {
      const int d0 = dc * 32 + g * 8;
      qf[j][dc] = d0 < D ? *(const u32x4*)(qp + (int64_t)qj * a.q_sn + d0) : u32x4{0, 0, 0, 0};
      df[j][dc] = d0 < D ? *(const u32x4*)(op + (int64_t)qj * a.o_sn + d0) : u32x4{0, 0, 0, 0};
    }
  }

  // Relative position: rel_h / rel_w of this workgroup's queries.
  const int gh = a.gh, gw = a.gw, G = gh + gw;
  const size_t stage_bytes = bwd_stage_bytes<D>(a);
  // General grids: rel_h/rel_w [64][G] (then dRel); after the key loop,
  // table slices and the Q tile.
  float* rel = (float*)(lds + stage_bytes);
  float* dacc = rel + (bwd_rows_rel_bytes<D>(a) - bwd_rows_acc_bytes(a)) / 4;
  const BwdWs wl = bwd_ws_layout(a);
  // This workgroup's partial slot; the 64-wide form first keeps dRelH^T
  // [gh][64] and dRelW^T [64][64] there (grid position major).
  float* pslot = ba.ws + wl.part + (int64_t)bid * wl.pstride;
  const int64_t bh = (int64_t)b * a.H + h;
  // [G][Nq] of this (batch item, head), in log2 units (the column kernel's form).
  float* ws_rel = ba.ws + wl.rel + bh * Nq * G;
  const uint16_t* rhp = (const uint16_t*)a.rh;
  const uint16_t* rwp = (const uint16_t*)a.rw;
  float wreg[RP == kBwdRelRow64 ? 16 : 1], wacc[RP == kBwdRelRow64 ? 16 : 1];
  const int GP = G | 1;  // general form: private rows of an odd stride (distinct banks per lane)
  // Small general grids: the one-hot key table [padded keys][kBwdAugRow]
  // where the general form keeps its private sums; the wave's B fragments of
  // rel_h / rel_w (columns g*8 .. g*8+7 of its query, divided by the scale,
  // as the element-type sum hi + lo, so the bias keeps about 16 bits), and
  // the dRel^T accumulators (rows x = 16 xb + 4g + i).
  uint16_t* Etab = (uint16_t*)dacc;
  u32x4 relq = u32x4{0, 0, 0, 0}, relq_lo = u32x4{0, 0, 0, 0};
  f32x4 drel[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if constexpr (RP == kBwdRelGeneral || RP == kBwdRelAug) {
    // rel_h[q][x] = Rh[qh - x + gh - 1] . q (rel_w likewise) from the
    // products G[m][q] = T[m] . q of every table row m with the wave's 16
    // queries on the matrix cores (query fragments as the B operand).  Lane
    // (query, g) then holds rows m = 16mb + 4g + i and keeps those its query
    // uses: each (query, x) comes from exactly one row.
    const int qh = fdiv(qi, a.fd_gw), qw = qi - qh * gw;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      const int nr = half ? 2 * gw - 1 : 2 * gh - 1, ng = half ? gw : gh, q0 = half ? qw : qh;
      const uint16_t* tp = half ? rwp : rhp;
      for (int mb = 0; mb < (nr + 15) / 16; ++mb) {
        const int m = min(mb * 16 + l16, nr - 1);
        f32x4 acc_t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < KCH; ++dc) {
          const int d0 = dc * 32 + g * 8;
          const u32x4 t = *(const u32x4*)(tp + (int64_t)m * D + (d0 < D ? d0 : 0));
          acc_t = E::mfma(d0 < D ? t : u32x4{0, 0, 0, 0}, qf[0][dc], acc_t);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mm = mb * 16 + g * 4 + i, x = q0 - mm + ng - 1;
          if (mm < nr && x >= 0 && x < ng) {
            const int col = half ? gh + x : x;
            rel[qloc * G + col] = acc_t[i];
            if (RP == kBwdRelGeneral && qrow < Nq) ws_rel[(int64_t)col * Nq + qrow] = acc_t[i] * kLog2e;
          }
        }
      }
    }
    if constexpr (RP == kBwdRelGeneral) {
      for (int e = tid; e < 256 * GP; e += 256) dacc[e] = 0.f;
    } else {
      const int erows = (Nk + 63) / 64 * 64;
      for (int e = tid * 8; e < erows * kBwdAugRow; e += 256 * 8) *(u32x4*)&Etab[e] = u32x4{0, 0, 0, 0};
      __syncthreads();  // the table is zero, and rel holds every column of the wave's queries
      for (int key = tid; key < Nk; key += 256) {
        const int kh = fdiv(key, a.fd_gw), kw = key - kh * gw;
        Etab[key * kBwdAugRow + kh] = E::one_bits();
        Etab[key * kBwdAugRow + gh + kw] = E::one_bits();
      }
      const float inv_scale = 1.f / a.scale;
      float ext[8], rem[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int x = g * 8 + e;
        ext[e] = x < G ? rel[qloc * G + x] * inv_scale : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        relq[e] = E::pack2(ext[2 * e], ext[2 * e + 1]);
        rem[2 * e] = ext[2 * e] - E::to_f((uint16_t)(relq[e] & 0xFFFFu));
        rem[2 * e + 1] = ext[2 * e + 1] - E::to_f((uint16_t)(relq[e] >> 16));
      }
      relq_lo = u32x4{E::pack2(rem[0], rem[1]), E::pack2(rem[2], rem[3]), E::pack2(rem[4], rem[5]),
                      E::pack2(rem[6], rem[7])};
      // The column kernel's copy: [B*H][Nq][hi 32 | lo 32] elements.
      if (qrow < Nq) {
        uint16_t* wq = (uint16_t*)(ba.ws + wl.rel) + (bh * Nq + qrow) * 64 + g * 8;
        *(u32x4*)wq = relq;
        *(u32x4*)(wq + 32) = relq_lo;
      }
    }
  } else if constexpr (RP == kBwdRelRow64) {
    // gw = 64: the workgroup's 64 queries are grid row qt, and a 64-key tile
    // is one grid row.  rel_h^T[kh][q] = Rh[qt + gh - 1 - kh] . q and
    // G_w[m][q] = Rw[m] . q (all 127 rows) on the matrix cores, with the
    // query fragments already in registers as the B operand.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int kh = mb * 16 + l16;
      f32x4 acc_h = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < KCH; ++dc) {
        const int d0 = dc * 32 + g * 8;
        const u32x4 af = kh < gh && d0 < D ? *(const u32x4*)(rhp + (int64_t)(qt + gh - 1 - kh) * D + d0)
                                           : u32x4{0, 0, 0, 0};
        acc_h = E::mfma(af, qf[0][dc], acc_h);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // lane (l16, g) holds rel_h[qloc][16mb + 4g + i]
        const int kh2 = mb * 16 + g * 4 + i;
        if (kh2 < gh) {
          if (qrow < Nq) ws_rel[(int64_t)kh2 * Nq + qrow] = acc_h[i] * kLog2e;
        }
      }
    }
    float* gwl = (float*)lds;  // [128][64] in the K/V stages (free until tile 0 is stored)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = mb * 16 + l16;
      f32x4 acc_w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < KCH; ++dc) {
        const int d0 = dc * 32 + g * 8;
        const u32x4 af = m < 127 && d0 < D ? *(const u32x4*)(rwp + (int64_t)m * D + d0) : u32x4{0, 0, 0, 0};
        acc_w = E::mfma(af, qf[0][dc], acc_w);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) gwl[(mb * 16 + g * 4 + i) * 64 + qloc] = acc_w[i];
    }
    __syncthreads();
    // rel_w[qloc][kw] = G_w[qloc - kw + 63][qloc] for this lane's key slots.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kw = (i >> 2) * 16 + g * 4 + (i & 3);
      wreg[i] = gwl[(qloc - kw + 63) * 64 + qloc] * kLog2e;  // log2 units
      if (qrow < Nq) ws_rel[(int64_t)(gh + kw) * Nq + qrow] = wreg[i];
      wacc[i] = 0.f;
    }
    __syncthreads();  // the stages are written below
  }

  zero_pad_cols<D>(Ks, 4, tid);  // both stages of K and V
  store_rows_regs<D>(Ks, kreg, tid);
  store_rows_regs<D>(Vs, vreg, tid);
  __syncthreads();

  const float c2 = a.scale * kLog2e;
  const int vt_row = g * 4 + (l16 >> 2), vt_col = 4 * (l16 & 3);
  // Pass 1 state of each query block (per lane: partial sums over its
  // keys, against the row maximum m shared by the four lane groups).
  float m[QB], l[QB], t[QB], L[QB], Dq[QB];
  // With the forward's O and log-sum-exp (attn_bwd_opt) the first pass is
  // not needed: L from lse (natural log -> log2), D = dO_i . O_i.
  const bool stats = ba.lse_in != nullptr;
  // Second-pass forms: the logits enter as scale*log2(e)*s + bias - L (yoff
  // = -L; 0 in the first pass), and dP accumulates onto -D (dinit), so that
  // P = exp2(y) and dS = P * dP take no further subtraction.
  float yoff[QB];
  f32x4 dinit[QB], acc[QB][CBD];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    m[j] = -INFINITY;
    l[j] = t[j] = L[j] = Dq[j] = 0.f;
    if (stats) {
      const int qj = min(qrow + 16 * j, Nq - 1);
      L[j] = ba.lse_in[(int64_t)(b * a.H + h) * Nq + qj] * kLog2e;
      const uint16_t* fop = (const uint16_t*)ba.fo + (int64_t)b * ba.fo_sb + (int64_t)h * ba.fo_sh +
                            (int64_t)qj * ba.fo_sn;
      float part = 0.f;
#pragma unroll
      for (int dc = 0; dc < KCH; ++dc) {
        const int d0 = dc * 32 + g * 8;
        if (d0 < D) {
          const u32x4 ov = *(const u32x4*)(fop + d0);
#pragma unroll
          for (int e = 0; e < 4; ++e) part = E::dot2(df[j][dc][e], ov[e], part);
        }
      }
      Dq[j] = sum_across_groups(part);
    }
    yoff[j] = stats ? -L[j] : 0.f;
    dinit[j] = stats ? f32x4{-Dq[j], -Dq[j], -Dq[j], -Dq[j]} : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < CBD; ++cb) acc[j][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int n_it = 2 * ntiles;
  const int it0 = stats ? ntiles : 0;  // tile 0 of the pass it starts with is in stage 0
  // One step of the key loop: iteration it of the two passes over the key
  // tiles (it < ntiles: statistics; it >= ntiles: gradients).  Each pass
  // runs as a loop of its own, so that the compiler keeps each pass's
  // state in place; the next tile's loads cross the pass boundary.
  // 64-wide form: rel_h of this query and the current tile's grid row, in
  // log2 units, from the workspace (written in the prologue, before the
  // barriers above); the next tile's value is loaded one tile ahead.
  float hcur = 0.f, hnext = 0.f;
  if constexpr (RP == kBwdRelRow64) hcur = ws_rel[qi];
  auto step = [&](int it, auto pass) {
    constexpr bool second = decltype(pass)::value;
    const int tile = second ? it - ntiles : it;
    const int st = (it - it0) & 1;
    const bool more = it + 1 < n_it;
    if (more) {  // the next tile's loads, in flight during this tile
      const int nt = it + 1 >= ntiles ? it + 1 - ntiles : it + 1;
      load_tile_regs<D>(kreg, kp, a.k_sn, nt * 64, Nk, koff);
      load_tile_regs<D>(vreg, vp, a.v_sn, nt * 64, Nk, voff);
      if constexpr (RP == kBwdRelRow64) hnext = ws_rel[(int64_t)nt * Nq + qi];
    }
    const uint16_t* Kt = Ks + st * TILE;
    const uint16_t* Vt = Vs + st * TILE;
    // The blocks of matrix products run at a raised wave priority, so a
    // wave that reaches them issues ahead of the others' vector work.
    __builtin_amdgcn_s_setprio(1);
    f32x4 s[QB][4], dp[QB][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        s[j][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[j][kb] = dinit[j];
      }
#pragma unroll
      for (int dc = 0; dc < KCH; ++dc) {
        const u32x4 ka = *(const u32x4*)&Kt[(kb * 16 + l16) * ROW + dc * 32 + g * 8];
        const u32x4 va = *(const u32x4*)&Vt[(kb * 16 + l16) * ROW + dc * 32 + g * 8];
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          s[j][kb] = E::mfma(ka, qf[j][dc], s[j][kb]);
          dp[j][kb] = E::mfma(va, df[j][dc], dp[j][kb]);
        }
      }
      if constexpr (RP == kBwdRelAug) {
        // + rel_h[q][kh] / scale + rel_w[q][kw] / scale: the key rows of the
        // one-hot table against the query's packed rel columns.
        const u32x4 ea = *(const u32x4*)&Etab[(tile * 64 + kb * 16 + l16) * kBwdAugRow + g * 8];
        s[0][kb] = E::mfma(ea, relq, s[0][kb]);
        s[0][kb] = E::mfma(ea, relq_lo, s[0][kb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    u32x4 sf[QB][2];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      float y[16];
      int kh_i[RP == kBwdRelGeneral ? 16 : 1], kw_i[RP == kBwdRelGeneral ? 16 : 1];
      // The 64-wide form: rel_h of this tile's grid row, with yoff folded in.
      float yrow = yoff[j];
      if constexpr (RP == kBwdRelRow64) yrow = hcur + yoff[j];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float sv = s[j][i >> 2][i & 3];
        if constexpr (RP == kBwdRelNone || RP == kBwdRelAug) {
          y[i] = fmaf(sv, c2, yoff[j]);
        } else if constexpr (RP == kBwdRelGeneral) {
          // Keys past Nk read the last key's entries (masked below).
          const int key = tile * 64 + (i >> 2) * 16 + g * 4 + (i & 3);
          const int kc = min(key, Nk - 1);
          kh_i[i] = fdiv(kc, a.fd_gw);
          kw_i[i] = kc - kh_i[i] * gw;
          const float bias = rel[qloc * G + kh_i[i]] + rel[qloc * G + gh + kw_i[i]];
          y[i] = fmaf(bias, kLog2e, fmaf(sv, c2, yoff[j]));
        } else {
          y[i] = fmaf(sv, c2, yrow) + wreg[i];
        }
      }
      // Keys past Nk only occur in the last tile (a uniform branch).
      if (tile * 64 + 64 > Nk) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (tile * 64 + (i >> 2) * 16 + g * 4 + (i & 3) >= Nk) y[i] = -INFINITY;
      }
      if constexpr (!second) {
        float mx = y[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, y[i]);
        const float mn = fmaxf(m[j], max_across_groups(mx));
        float ps = 0.f, pd = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(y[i] - mn);
          ps += e;
          pd = fmaf(e, dp[j][i >> 2][i & 3], pd);
        }
        const float alpha = __builtin_amdgcn_exp2f(m[j] - mn);  // 0 on the first tile
        l[j] = fmaf(l[j], alpha, ps);
        t[j] = fmaf(t[j], alpha, pd);
        m[j] = mn;
        if (it == ntiles - 1) {
          const float lt = sum_across_groups(l[j]);
          L[j] = m[j] + __builtin_amdgcn_logf(lt);  // log2 of the row sum
          Dq[j] = sum_across_groups(t[j]) / lt;
          yoff[j] = -L[j];
          dinit[j] = f32x4{-Dq[j], -Dq[j], -Dq[j], -Dq[j]};
        }
      } else {
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = __builtin_amdgcn_exp2f(y[i]) * dp[j][i >> 2][i & 3];
        if constexpr (RP == kBwdRelGeneral) {
          // Private sums of this lane (keys past Nk have dS = 0).
          float* my = dacc + tid * GP;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            my[kh_i[i]] += ds[i];
            my[gh + kw_i[i]] += ds[i];
          }
        } else if constexpr (RP == kBwdRelRow64) {
          float rs = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            rs += ds[i];
            wacc[i] += ds[i];
          }
          rs = sum_across_groups(rs);
          if (g == 0) pslot[tile * 64 + qloc] = rs;
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          sf[j][kc] = u32x4{E::pack2(ds[kc * 8 + 0], ds[kc * 8 + 1]), E::pack2(ds[kc * 8 + 2], ds[kc * 8 + 3]),
                            E::pack2(ds[kc * 8 + 4], ds[kc * 8 + 5]), E::pack2(ds[kc * 8 + 6], ds[kc * 8 + 7])};
        if constexpr (RP == kBwdRelAug) {
          // dRel^T[x][q] += sum_key E[key][x] dS[q][key]: the table by
          // transposing reads (key order as in sf), like K^T for dQ.
#pragma unroll
          for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int xb = 0; xb < 2; ++xb) {
              const uint16_t* ep = Etab + (tile * 64 + kc * 32 + vt_row) * kBwdAugRow + xb * 16 + vt_col;
              const u32x2 lo = lds_read_tr16(ep);
              const u32x2 hi = lds_read_tr16(ep + 16 * kBwdAugRow);
              drel[xb] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, sf[j][kc], drel[xb]);
            }
        }
      }
    }
    if constexpr (second) {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int cb = 0; cb < CBD; ++cb) {
          const uint16_t* ptr = Kt + (kc * 32 + vt_row) * ROW + cb * 16 + vt_col;
          const u32x2 lo = lds_read_tr16(ptr);
          const u32x2 hi = lds_read_tr16(ptr + 16 * ROW);
#pragma unroll
          for (int j = 0; j < QB; ++j) acc[j][cb] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, sf[j][kc], acc[j][cb]);
        }
      __builtin_amdgcn_s_setprio(0);
    }
    if (more) {
      // Stage st^1 was last read in the previous tile, before the barrier
      // that ended it; this tile's reads of stage st end at the barrier below.
      store_rows_regs<D>(Ks + (st ^ 1) * TILE, kreg, tid);
      store_rows_regs<D>(Vs + (st ^ 1) * TILE, vreg, tid);
      if constexpr (RP == kBwdRelRow64) hcur = hnext;
    }
    __syncthreads();
  };
  wait_all_vmem();
  for (int it = it0; it < ntiles; ++it) step(it, std::false_type{});
  for (int it = ntiles; it < n_it; ++it) step(it, std::true_type{});
  float* wsL = ba.ws + (int64_t)(b * a.H + h) * Nq;
  float* wsD = wsL + (int64_t)a.B * a.H * Nq;
  f32x4 bq[CBD];  // bias path of dQ (already in final units)
#pragma unroll
  for (int cb = 0; cb < CBD; ++cb) bq[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (RP != kBwdRelNone) {
    const int RH = 2 * gh - 1, RW = 2 * gw - 1, RT = RH + RW;
    // dRel of this workgroup's queries: general grids sum the four lane
    // groups' private rows into `rel` [64][G]; the row form has dRelH^T in
    // its partial slot and adds dRelW^T from registers.
    if constexpr (RP == kBwdRelAug) {
      // Each wave's own queries (rel is not read after the prologue).
#pragma unroll
      for (int xb = 0; xb < 2; ++xb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int x = xb * 16 + g * 4 + i;
          if (x < G) rel[qloc * G + x] = drel[xb][i];
        }
    } else if constexpr (RP == kBwdRelGeneral) {
      for (int e = tid; e < 64 * G; e += 256) {
        const int ql = e / G, x = e - ql * G;
        const int base = (ql >> 4) * 64 + (ql & 15);
        rel[e] = ((dacc[base * GP + x] + dacc[(base + 16) * GP + x]) + dacc[(base + 32) * GP + x]) +
                 dacc[(base + 48) * GP + x];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) pslot[(gh + (i >> 2) * 16 + g * 4 + (i & 3)) * 64 + qloc] = wacc[i];
    }
    auto d_relh = [&](int ql, int x) { return RP != kBwdRelRow64 ? rel[ql * G + x] : pslot[x * 64 + ql]; };
    auto d_relw = [&](int ql, int x) { return RP != kBwdRelRow64 ? rel[ql * G + gh + x] : pslot[(gh + x) * 64 + ql]; };
    __syncthreads();
    // Coefficients A[r][i] (element type) in the free K/V stages: the weight
    // of table row r (Rh rows, then Rw rows) in query i's bias; zero for
    // rows RT .. AR-1 and queries past Nq.
    const int AR = bwd_rel_arows(a);
    uint16_t* Am = (uint16_t*)lds;  // [AR][kBwdARow]
    for (int e = tid; e < AR * 64; e += 256) {
      const int r = e >> 6, ql = e & 63, qr = qt * 64 + ql;
      float v = 0.f;
      if (r < RT && qr < Nq) {
        const int qh = fdiv(qr, a.fd_gw), qw = qr - qh * gw;
        if (r < RH) {
          const int x = qh + gh - 1 - r;
          if (x >= 0 && x < gh) v = d_relh(ql, x);
        } else {
          const int x = qw + gw - 1 - (r - RH);
          if (x >= 0 && x < gw) v = d_relw(ql, x);
        }
      }
      Am[r * kBwdARow + ql] = (uint16_t)(E::pack2(v, 0.f) & 0xFFFF);
    }
    __syncthreads();  // `rel`, `dacc` and the slot's dRel are free: table slices, then the Q tile go there
    // Bias path of dQ on the matrix cores, one table slice at a time:
    //   dQ_bias^T[c][i] = sum_r T^T[c][r] A[r0 + r][i]  (T = Rh, r0 = 0; T = Rw, r0 = RH).
    // Both operands by transposing reads (the slice staged with rows padded
    // to 32 by zeros, A as it stands), so their K orders agree; the result
    // has the layout of the dQ accumulators.
    {
      constexpr int TR = bwd_rel_tab_row<D>();
      const int TS = bwd_rel_tab_rows(a);
      uint16_t* Tb = (uint16_t*)rel;
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        const int nr = half ? RW : RH, r0 = half ? RH : 0;
        const uint16_t* src = half ? rwp : rhp;
#pragma unroll 1
        for (int s0 = 0; s0 < nr; s0 += TS) {
          const int ns = min(TS, nr - s0), nrp = bwd_up32(ns);
          for (int e = tid * 8; e < nrp * TR; e += 256 * 8) {
            const int row = e / TR, col = e - row * TR;
            *(u32x4*)&Tb[e] = row < ns && col < D ? *(const u32x4*)(src + (s0 + row) * D + col) : u32x4{0, 0, 0, 0};
          }
          __syncthreads();
          for (int kc = 0; kc < nrp / 32; ++kc) {
            const uint16_t* aptr = Am + (r0 + s0 + kc * 32 + vt_row) * kBwdARow + wave * 16 + vt_col;
            const u32x2 blo = lds_read_tr16(aptr), bhi = lds_read_tr16(aptr + 16 * kBwdARow);
#pragma unroll
            for (int cb = 0; cb < CBD; ++cb) {
              const uint16_t* tptr = Tb + (kc * 32 + vt_row) * TR + cb * 16 + vt_col;
              const u32x2 tlo = lds_read_tr16(tptr), thi = lds_read_tr16(tptr + 16 * TR);
              bq[cb] = E::mfma(u32x4{tlo[0], tlo[1], thi[0], thi[1]}, u32x4{blo[0], blo[1], bhi[0], bhi[1]}, bq[cb]);
            }
          }
          __syncthreads();
        }
      }
    }
    const int RB = (RT + 15) / 16;
    uint16_t* Qs = (uint16_t*)rel;
    {
      u32x4 qreg[C::CPT];
      load_rows_regs<D>(qreg, qp, a.q_sn, qt * 64, Nq, tid);
      zero_pad_cols<D>(Qs, 1, tid);
      store_rows_regs<D>(Qs, qreg, tid);
    }
    __syncthreads();
    // part^T[c][r] = sum_i Q[i][c] A[r][i]: A operand Q^T by transposing
    // reads of the Q tile, B operand A^T (lane = table row r), both in the
    // query order the transposing reads produce.
    float* part = pslot;
    for (int rb = wave; rb < RB; rb += 4) {
#pragma unroll
      for (int cb = 0; cb < CBD; ++cb) {
        f32x4 pr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const uint16_t* ptr = Qs + (kc * 32 + vt_row) * ROW + cb * 16 + vt_col;
          const u32x2 lo = lds_read_tr16(ptr);
          const u32x2 hi = lds_read_tr16(ptr + 16 * ROW);
          // B operand in the key order of the transposing reads: slot j of
          // lane group g is query kc*32 + (j/4)*16 + 4g + j%4.
          const uint16_t* arow = Am + (rb * 16 + l16) * kBwdARow + kc * 32 + g * 4;
          const u32x2 alo = *(const u32x2*)arow, ahi = *(const u32x2*)(arow + 16);
          pr = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, u32x4{alo[0], alo[1], ahi[0], ahi[1]}, pr);
        }
        const int r = rb * 16 + l16, c0 = cb * 16 + g * 4;
        if (r < RT && c0 < D) *(f32x4*)&part[(int64_t)r * D + c0] = pr;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int qr = qrow + 16 * j;
    if (qr < Nq) {
      if (g == 0) {
        wsL[qr] = L[j];
        wsD[qr] = Dq[j];
      }
      uint16_t* dq = (uint16_t*)ba.dq + (int64_t)b * ba.dq_sb + (int64_t)h * ba.dq_sh + (int64_t)qr * ba.dq_sn;
#pragma unroll
      for (int cb = 0; cb < CBD; ++cb) {
        const int c0 = cb * 16 + g * 4;
        if (c0 < D) {
          const f32x4 v = acc[j][cb] * a.scale + (j == 0 ? bq[cb] : f32x4{0.f, 0.f, 0.f, 0.f});
          *(u32x2*)(dq + c0) = u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
        }
      }
    }
  }
}

// RP: as for the row kernel; the bias of (query i, this lane's key) comes
// from the rel_h / rel_w rows the row kernel stored: for general grids all
// gh + gw columns staged per query tile in log2 units ([columns][64]
// floats); in the 64-wide form the key tile's rel_h column joins the staged
// log-sum-exp and each lane reads its own rel_w column.
//
// KB: 16-key blocks per wave (a workgroup covers 64 KB keys).  With KB = 2
// every fragment read from the staged Q / dO tiles feeds two products, which
// halves the LDS reads per matrix instruction (no relative position).
template <class E, int D, int RP = kBwdRelNone, int KB = 1>
__global__ __launch_bounds__(256) void attn_bwd_cols(AttnBwdArgs ba) {
  static_assert(KB == 1 || (KB == 2 && RP == kBwdRelNone), "two key blocks per wave: no relative position");
  using C = BwdTileCfg<D>;
  constexpr int KCH = C::KCH, CBD = C::CBD, ROW = C::ROW, TILE = C::TILE;
  const AttnArgs& a = ba.a;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* Qs = (uint16_t*)lds;  // [2][64][ROW]
  uint16_t* Os = Qs + 2 * TILE;   // dO, [2][64][ROW]
  float* Ls = (float*)(Os + 2 * TILE);  // [2][64]
  float* Ds = Ls + 2 * 64;              // [2][64]
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int bid = xcd_logical_id(__builtin_amdgcn_workgroup_id_x(), a.n_blocks);
  const int kt_div = fdiv(bid, a.fd_qt);  // key tiles
  const int kt = bid - kt_div * a.n_qtiles;
  const int b = fdiv(kt_div, a.fd_h), h = kt_div - b * a.H;
  const int Nq = a.Nq, Nk = a.Nk;
  const int krow0 = kt * 64 * KB + wave * 16 * KB + l16;  // key of block kb: krow0 + 16 kb
  const int ki = min(krow0, Nk - 1);
  const uint16_t* qp = (const uint16_t*)a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
  const uint16_t* kp = (const uint16_t*)a.k + (int64_t)b * a.k_sb + (int64_t)h * a.k_sh;
  const uint16_t* vp = (const uint16_t*)a.v + (int64_t)b * a.v_sb + (int64_t)h * a.v_sh;
  const uint16_t* op = (const uint16_t*)a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;  // dO
  const float* wsL = ba.ws + (int64_t)(b * a.H + h) * Nq;
  const float* wsD = wsL + (int64_t)a.B * a.H * Nq;
  const int ntiles = (Nq + 63) / 64;
  // Relative position: staged columns NC, this lane's two of them.
  const int gh = a.gh, G = gh + a.gw;
  const int NC = bwd_cols_rel_cols(a);
  float* Rst = Ds + 2 * 64;  // [2][NC][64]
  const float* ws_rel = ba.ws + bwd_ws_layout(a).rel + ((int64_t)b * a.H + h) * Nq * G;
  // Columns of this lane's key: rel_h column kh and rel_w column gh + kw.
  // General grids stage all columns per query tile (each is shared by the
  // keys of one grid row or column).  The 64-wide form folds the tile's
  // rel_h column (grid row kt) into the staged L and reads the lane's own
  // rel_w column straight from the workspace (one consumer per entry).
  int xh = 0, xw = 0;
  if constexpr (RP != kBwdRelNone) {
    const int kh = fdiv(ki, a.fd_gw), kw = ki - kh * a.gw;
    xh = kh;
    xw = gh + kw;
  }
  // The one-hot table's form: E[key][x] of this lane's key as the B
  // fragment of the bias product (slots x = g*8 .. g*8+7), and the staged
  // packed rel rows [2][64][kBwdAugQRow] of the query tile.
  u32x4 ef = u32x4{0, 0, 0, 0};
  if constexpr (RP == kBwdRelAug) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = g * 8 + 2 * e;
      const uint32_t lo = x == xh || x == xw ? E::one_bits() : 0u;
      const uint32_t hi = x + 1 == xh || x + 1 == xw ? E::one_bits() : 0u;
      ef[e] = lo | hi << 16;
    }
  }
  uint16_t* Rq = (uint16_t*)Rst;
  const uint16_t* ws_relq =
      RP == kBwdRelAug ? (const uint16_t*)(ba.ws + bwd_ws_layout(a).rel) + ((int64_t)b * a.H + h) * Nq * 64 : nullptr;
  u32x4 rqreg[2];
  constexpr int RC = RP == kBwdRelGeneral ? (kBwdRelMaxCols * 64 + 255) / 256 : 1;
  f32x4 wv[RP == kBwdRelRow64 ? 4 : 1];  // 64-wide form: rel_w column xw, a tile's 64 queries
  auto load_w = [&](int t) {
    if constexpr (RP == kBwdRelRow64) {
      // Nq = 64 gh: whole tiles; 16-byte aligned in the workspace.
      const float* col = ws_rel + (int64_t)xw * Nq + t * 64 + g * 4;
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) wv[qb] = *(const f32x4*)(col + qb * 16);
    }
  };
  float rreg[RC];
  u32x4 qreg[C::CPT], oreg[C::CPT];
  uint32_t qoff[C::CPT], ooff[C::CPT];
  tile_chunk_offsets<D>(qoff, a.q_sn, tid);
  tile_chunk_offsets<D>(ooff, a.o_sn, tid);
  float lreg = 0.f, dreg = 0.f, hreg = 0.f;
  // Query rows past Nq read as zero (Q, dO, their D); their L is set to
  // +inf when staged, so that P = 0 for them whatever their bias.
  auto load_tile = [&](int t) {
    load_tile_regs<D>(qreg, qp, a.q_sn, t * 64, Nq, qoff);
    load_tile_regs<D>(oreg, op, a.o_sn, t * 64, Nq, ooff);
    if (tid < 64) {
      const uint32_t nb = (uint32_t)(Nq - t * 64) * 4;
      lreg = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(wsL + t * 64, nb), tid * 4, 0, 0));
      dreg = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(wsD + t * 64, nb), tid * 4, 0, 0));
      if constexpr (RP == kBwdRelRow64)
        hreg = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(ws_rel + (int64_t)kt * Nq + t * 64, nb), tid * 4, 0, 0));
    }
    if constexpr (RP == kBwdRelAug) {
      // 64 rows of 128 bytes; rows past Nq read as zero.
      const auto rr = buffer_rsrc(ws_relq + (int64_t)t * 64 * 64, (uint32_t)(Nq - t * 64) * 128);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + i * 256;
        rqreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rr, (uint32_t)c * 16, 0, 0);
      }
    }
    if constexpr (RP == kBwdRelGeneral) {
      // [G][Nq] floats of this (batch item, head): at most 84 x 1764.
      const auto rr = buffer_rsrc(ws_rel, (uint32_t)(G * Nq) * 4);
#pragma unroll
      for (int c = 0; c < RC; ++c) {
        // Column x of the stage is rel_h / rel_w column x.  Rows past Nq
        // read another column's finite entries or zero; their P is 0.
        const int e = tid + c * 256, x = e >> 6, q = t * 64 + (e & 63);
        if (e < 64 * NC) rreg[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)(x * Nq + q) * 4, 0, 0));
      }
    }
  };
  // L and D are staged negated: the exponent is scale*log2(e)*s + bias - L
  // with one FMA, and dP accumulates onto -D.  The bias terms come in log2
  // units; the 64-wide form's rel_h term is part of the staged -L.
  auto store_tile = [&](int st, int t) {
    store_rows_regs<D>(Qs + st * TILE, qreg, tid);
    store_rows_regs<D>(Os + st * TILE, oreg, tid);
    if (tid < 64) {
      Ls[st * 64 + tid] = t * 64 + tid < Nq ? hreg - lreg : -INFINITY;
      Ds[st * 64 + tid] = -dreg;
    }
    if constexpr (RP == kBwdRelGeneral) {
#pragma unroll
      for (int c = 0; c < RC; ++c) {
        const int e = tid + c * 256;
        if (e < 64 * NC) Rst[st * 64 * NC + e] = rreg[c];
      }
    }
    if constexpr (RP == kBwdRelAug) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + i * 256;  // row c / 8, chunk c % 8
        *(u32x4*)&Rq[st * 64 * kBwdAugQRow + (c >> 3) * kBwdAugQRow + (c & 7) * 8] = rqreg[i];
      }
    }
  };
  load_tile(0);
  load_w(0);
  // K and V rows of this lane's keys as B operands (lane = key column).
  u32x4 kf[KB][KCH], vf[KB][KCH];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int kr = min(krow0 + 16 * kb, Nk - 1);
#pragma unroll
    for (int dc = 0; dc < KCH; ++dc) {
      const int d0 = dc * 32 + g * 8;
      kf[kb][dc] = d0 < D ? *(const u32x4*)(kp + (int64_t)kr * a.k_sn + d0) : u32x4{0, 0, 0, 0};
      vf[kb][dc] = d0 < D ? *(const u32x4*)(vp + (int64_t)kr * a.v_sn + d0) : u32x4{0, 0, 0, 0};
    }
  }
  zero_pad_cols<D>(Qs, 4, tid);  // both stages of Q and dO
  store_tile(0, 0);
  __syncthreads();
  const float c2 = a.scale * kLog2e;
  const int vt_row = g * 4 + (l16 >> 2), vt_col = 4 * (l16 & 3);
  f32x4 dk[KB][CBD], dv[KB][CBD];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int cb = 0; cb < CBD; ++cb) dk[kb][cb] = dv[kb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  wait_all_vmem();
  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);  // in flight during this tile
    const uint16_t* Qt = Qs + st * TILE;
    const uint16_t* Ot = Os + st * TILE;
    const float* Lt = Ls + st * 64;
    const float* Dt = Ds + st * 64;
    // S = Q K^T and dP = dO V^T - D: rows are queries qb*16 + g*4 + r, the
    // column is this lane's key of block kb.
    __builtin_amdgcn_s_setprio(1);
    f32x4 s[KB][4], dp[KB][4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const f32x4 nD = *(const f32x4*)&Dt[qb * 16 + g * 4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kb][qb] = nD;
      }
#pragma unroll
      for (int dc = 0; dc < KCH; ++dc) {
        const u32x4 qa = *(const u32x4*)&Qt[(qb * 16 + l16) * ROW + dc * 32 + g * 8];
        const u32x4 oa = *(const u32x4*)&Ot[(qb * 16 + l16) * ROW + dc * 32 + g * 8];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[kb][qb] = E::mfma(qa, kf[kb][dc], s[kb][qb]);
          dp[kb][qb] = E::mfma(oa, vf[kb][dc], dp[kb][qb]);
        }
      }
      if constexpr (RP == kBwdRelAug) {
        // + (rel_h[q][kh] + rel_w[q][kw]) / scale, high and low parts.
        const uint16_t* rq = Rq + st * 64 * kBwdAugQRow + (qb * 16 + l16) * kBwdAugQRow + g * 8;
        s[0][qb] = E::mfma(*(const u32x4*)rq, ef, s[0][qb]);
        s[0][qb] = E::mfma(*(const u32x4*)(rq + 32), ef, s[0][qb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    u32x4 pf[KB][2], sf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float p[16], ds[16];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const f32x4 nL = *(const f32x4*)&Lt[qb * 16 + g * 4];
        f32x4 bias = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (RP == kBwdRelGeneral) {
          const float* rs = Rst + st * 64 * NC + qb * 16 + g * 4;
          bias = *(const f32x4*)(rs + xh * 64) + *(const f32x4*)(rs + xw * 64);
        } else if constexpr (RP == kBwdRelRow64) {
          bias = wv[qb];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float y = fmaf(s[kb][qb][r], c2, nL[r]);
          if constexpr (RP == kBwdRelGeneral || RP == kBwdRelRow64) y += bias[r];
          const float pv = __builtin_amdgcn_exp2f(y);
          p[qb * 4 + r] = pv;
          ds[qb * 4 + r] = pv * dp[kb][qb][r];
        }
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        pf[kb][kc] = u32x4{E::pack2(p[kc * 8 + 0], p[kc * 8 + 1]), E::pack2(p[kc * 8 + 2], p[kc * 8 + 3]),
                           E::pack2(p[kc * 8 + 4], p[kc * 8 + 5]), E::pack2(p[kc * 8 + 6], p[kc * 8 + 7])};
        sf[kb][kc] = u32x4{E::pack2(ds[kc * 8 + 0], ds[kc * 8 + 1]), E::pack2(ds[kc * 8 + 2], ds[kc * 8 + 3]),
                           E::pack2(ds[kc * 8 + 4], ds[kc * 8 + 5]), E::pack2(ds[kc * 8 + 6], ds[kc * 8 + 7])};
      }
    }
    if (more) load_w(t + 1);  // the values of this tile are used: the next tile's, in flight from here
    // dV^T += dO^T P and dK^T += Q^T dS (transposing reads of the tiles).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int cb = 0; cb < CBD; ++cb) {
        const uint16_t* optr = Ot + (kc * 32 + vt_row) * ROW + cb * 16 + vt_col;
        const uint16_t* qptr = Qt + (kc * 32 + vt_row) * ROW + cb * 16 + vt_col;
        const u32x2 ol = lds_read_tr16(optr), oh = lds_read_tr16(optr + 16 * ROW);
        const u32x2 ql = lds_read_tr16(qptr), qh = lds_read_tr16(qptr + 16 * ROW);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          dv[kb][cb] = E::mfma(u32x4{ol[0], ol[1], oh[0], oh[1]}, pf[kb][kc], dv[kb][cb]);
          dk[kb][cb] = E::mfma(u32x4{ql[0], ql[1], qh[0], qh[1]}, sf[kb][kc], dk[kb][cb]);
        }
      }
    __builtin_amdgcn_s_setprio(0);
    if (more) store_tile(st ^ 1, t + 1);  // stage st^1 was last read before the previous barrier
    __syncthreads();
  }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int krow = krow0 + 16 * kb;
    if (krow < Nk) {
      uint16_t* dkp = (uint16_t*)ba.dk + (int64_t)b * ba.dk_sb + (int64_t)h * ba.dk_sh + (int64_t)krow * ba.dk_sn;
      uint16_t* dvp = (uint16_t*)ba.dv + (int64_t)b * ba.dv_sb + (int64_t)h * ba.dv_sh + (int64_t)krow * ba.dv_sn;
#pragma unroll
      for (int cb = 0; cb < CBD; ++cb) {
        const int c0 = cb * 16 + g * 4;
        if (c0 < D) {
          const f32x4 k4 = dk[kb][cb] * a.scale, v4 = dv[kb][cb];
          *(u32x2*)(dkp + c0) = u32x2{E::pack2(k4[0], k4[1]), E::pack2(k4[2], k4[3])};
          *(u32x2*)(dvp + c0) = u32x2{E::pack2(v4[0], v4[1]), E::pack2(v4[2], v4[3])};
        }
      }
    }
  }
}

// Relative-position table gradients: out[o] = sum over the row-kernel
// workgroups p of part[p * stride + o] (o = r*D + c over the stacked
// [Rh; Rw] rows), in two fixed-order stages (bitwise deterministic):
// attn_bwd_part_reduce sums slice s of the parts, p in [s*P/S, (s+1)*P/S),
// into sums[s][o] (out itself when S = 1), and attn_bwd_part_final adds the
// S slices in order.  Slicing lets small tables still fill the chip.
// Within a slice, one workgroup of 16 waves per 64 outputs: wave w adds
// p = w, w+16, ... in order, then the 16 partial sums are added in a fixed
// order.  The loads of 8 parts are issued together before they are added
// (in the same order), so each wave keeps 8 in flight.  (Templates only so
// that every compiled instance may carry its copy.)
template <int>
__global__ __launch_bounds__(1024) void attn_bwd_part_reduce(const float* part, float* sums, int n_out, int n_part,
                                                              int64_t stride, int S) {
  __shared__ float red[16][64];
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63, w = tid >> 6;
  const int o = __builtin_amdgcn_workgroup_id_x() * 64 + lane;
  const int sl = __builtin_amdgcn_workgroup_id_y();  // slice, < S
  const int p0 = (int)((int64_t)n_part * sl / S), p1 = (int)((int64_t)n_part * (sl + 1) / S);
  float acc = 0.f;
  if (o < n_out) {
    const float* src = part + o;
    const size_t step = (size_t)16 * stride;
    int p = p0 + w;
    for (; p + 7 * 16 < p1; p += 8 * 16) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = src[(size_t)p * stride + j * step];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += v[j];
    }
    for (; p < p1; p += 16) acc += src[(size_t)p * stride];
  }
  red[w][lane] = acc;
  __syncthreads();
  if (w == 0 && o < n_out) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) t += red[j][lane];
    sums[(int64_t)sl * n_out + o] = t;
  }
}

template <int>
__global__ __launch_bounds__(256) void attn_bwd_part_final(const float* sums, float* out, int n_out, int S) {
  const int o = __builtin_amdgcn_workgroup_id_x() * 256 + __builtin_amdgcn_workitem_id_x();
  if (o < n_out) {
    float t = 0.f;
    for (int s = 0; s < S; ++s) t += sums[(int64_t)s * n_out + o];
    out[o] = t;
  }
}

}  // namespace attn

#endif  // ATTN_BWD_H_
