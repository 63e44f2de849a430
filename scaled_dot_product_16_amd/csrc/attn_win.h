// Short-sequence attention (windows of up to 64 tokens) on gfx950.
//
// Swin-style window attention has many small, independent (window, head)
// units: 49 tokens each for 7x7 windows.  One wave owns one unit and keeps
// all of it on chip: Q and K are loaded straight from memory into MFMA
// operand registers, V is staged in a per-wave LDS slice for the
// transposing read, the 64x64 score tile (keys past N start from -inf) lives
// in registers, and the softmax needs no running rescale because the whole
// key range is one tile.  Table bias indices, region labels and the image
// addressing of the window partition and cyclic shift (Swin talk, sections 1
// and 2) are computed from per-lane token coordinates that are the same for
// every unit.
#ifndef ATTN_WIN_H_
#define ATTN_WIN_H_

#include "attn_mfma.h"

namespace attn {

constexpr int kWinWaves = 4;

template <int D>
struct WinCfg {
  static constexpr int NT = kWinWaves * 64;
  static constexpr int KCH = (D + 31) / 32;
  static constexpr int DK = KCH * 32;
  static constexpr int CB = (D + 15) / 16;
  static constexpr int DV = CB * 16;
  static constexpr int KROW = DK + 8;
  static constexpr int VROW = DV + 8;
  static constexpr int RCH = D / 8;
  static constexpr int NCH = 64 * RCH;               // 16-byte chunks of a 64-token tile
  static constexpr int CPT = (NCH + NT - 1) / NT;    // per thread
  static constexpr size_t KV_BYTES = (size_t)64 * (KROW + VROW) * 2;
};

inline size_t win_lds_bytes(const AttnArgs& a, size_t kv_bytes) {
  size_t n = kv_bytes + 64 * 4;  // per-key index data
  if (a.bias_kind == ATTN_BIAS_TABLE) n += (size_t)(2 * a.gh - 1) * (2 * a.gw - 1) * 4;
  return n;
}

// Per-unit window placement (image layout and region labels).
struct WinPos {
  int img;     // image index (image layout)
  int y0, x0;  // shifted-image origin of the window
};

__device__ __forceinline__ WinPos win_pos(const AttnArgs& a, int b) {
  WinPos p;
  const int nw = a.nw ? a.nw : 1;
  p.img = b / nw;
  const int w = b - p.img * nw;
  const int wy = a.nwx ? w / a.nwx : 0;
  const int wx = w - wy * a.nwx;
  p.y0 = wy * a.win_h;
  p.x0 = wx * a.win_w;
  return p;
}

// Element offset of window token (ty, tx) inside one (image, head) slice.
__device__ __forceinline__ uint32_t win_tok_off(const AttnArgs& a, const WinPos& p, int ty, int tx,
                                                int64_t sn) {
  int y = p.y0 + ty + a.shift_h;
  if (y >= a.img_h) y -= a.img_h;
  int x = p.x0 + tx + a.shift_w;
  if (x >= a.img_w) x -= a.img_w;
  return (uint32_t)(y * a.img_w + x) * (uint32_t)sn;
}

__device__ __forceinline__ int win_region(const AttnArgs& a, const WinPos& p, int ty, int tx) {
  const int y = p.y0 + ty, x = p.x0 + tx;
  const int ry = y < a.img_h - a.win_h ? 0 : (y < a.img_h - a.shift_h ? 1 : 2);
  const int rx = x < a.img_w - a.win_w ? 0 : (x < a.img_w - a.shift_w ? 1 : 2);
  return 3 * ry + rx;
}

// One workgroup = one (batch item, head) unit of at most 64 tokens; wave w
// owns queries 16w .. 16w+15.  MASKK: ATTN_MASK_NONE / _ADDITIVE /
// _SHIFT_REGIONS.
template <class E, int D, int BIAS, int MASKK>
__global__ __launch_bounds__(kWinWaves * 64) void attn_fwd_win(AttnArgs a) {
  using C = WinCfg<D>;
  constexpr int NT = C::NT, KCH = C::KCH, DK = C::DK, CB = C::CB, DV = C::DV, KROW = C::KROW,
                VROW = C::VROW, RCH = C::RCH, NCH = C::NCH, CPT = C::CPT;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* Ks = (uint16_t*)lds;        // [64][KROW]
  uint16_t* Vs = Ks + 64 * KROW;        // [64][VROW]
  int* kinfo = (int*)(lds + C::KV_BYTES);            // per key: table offset | region << 24
  float* tbl = (float*)(lds + C::KV_BYTES + 64 * 4);  // this head's table column, log2 units

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int H = a.H, N = a.Nq, Nk = a.Nk;
  const int unit = blockIdx.x;
  const int b = unit / H, h = unit - (unit / H) * H;

  // Token t < 64 of a window -> (row, column) for a row length n <= 1024: the
  // float quotient (t + 0.5) / n is within 2e-5 of the exact value and at
  // least 0.5 / n away from an integer, so truncation is exact.
  const float inv_ww = 1.f / (float)(a.win_w > 0 ? a.win_w : 1);
  const float inv_gw = 1.f / (float)(a.gw > 0 ? a.gw : 1);
  auto div_small = [](int t, float inv) { return (int)(((float)t + 0.5f) * inv); };
  auto split = [&](int t, int& ty, int& tx) {
    ty = div_small(t, inv_ww);
    tx = t - ty * a.win_w;
  };
  const WinPos pos = win_pos(a, b);
  const int bimg = a.image ? pos.img : b;
  auto row_off = [&](int t, int64_t sn) -> uint32_t {
    if (!a.image) return (uint32_t)t * (uint32_t)sn;
    int ty, tx;
    split(t, ty, tx);
    return win_tok_off(a, pos, ty, tx, sn);
  };
  const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)bimg * a.q_sb + (int64_t)h * a.q_sh);
  const uint16_t* kp = (const uint16_t*)a.k + ((int64_t)bimg * a.k_sb + (int64_t)h * a.k_sh);
  const uint16_t* vp = (const uint16_t*)a.v + ((int64_t)bimg * a.v_sb + (int64_t)h * a.v_sh);
  uint16_t* op = (uint16_t*)a.o + ((int64_t)bimg * a.o_sb + (int64_t)h * a.o_sh);

  // Global loads first.  Token rows past N are clamped to the last token, so
  // every load is unconditional; those keys start from -inf below, so their
  // probabilities are exactly zero and their finite values never reach O.
  u32x4 kreg[CPT], vreg[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = min(tid + c * NT, NCH - 1);
    const int key = min(ch / RCH, Nk - 1);
    const uint32_t col = (uint32_t)((ch % RCH) * 8);
    kreg[c] = *(const u32x4*)(kp + (row_off(key, a.k_sn) + col));
    vreg[c] = *(const u32x4*)(vp + (row_off(key, a.v_sn) + col));
  }
  const int q_tok = min(wave * 16 + l16, N - 1);
  const uint32_t q_off = row_off(q_tok, a.q_sn);
  u32x4 qf[KCH];
#pragma unroll
  for (int dc = 0; dc < KCH; ++dc) {
    const int d0 = dc * 32 + g * 8;
    qf[dc] = d0 < D ? *(const u32x4*)(qp + (q_off + (uint32_t)d0)) : u32x4{0, 0, 0, 0};
  }
  if constexpr (BIAS == ATTN_BIAS_TABLE) {
    const int n = (2 * a.gh - 1) * (2 * a.gw - 1);
    for (int r = tid; r < n; r += NT) tbl[r] = load_elem<E>(a.table, (int64_t)r * H + h) * kLog2e;
  }
  const bool regions = MASKK == ATTN_MASK_SHIFT_REGIONS &&
                       (pos.y0 + a.win_h > a.img_h - a.win_h || pos.x0 + a.win_w > a.img_w - a.win_w);
  if (tid < 64) {
    const int j = min(tid, Nk - 1);
    int info = 0;
    if constexpr (BIAS == ATTN_BIAS_TABLE) {
      const int kh = div_small(j, inv_gw), kw = j - kh * a.gw;
      info = kh * (2 * a.gw - 1) + kw;
    }
    if (regions) {
      int ty, tx;
      split(j, ty, tx);
      info |= win_region(a, pos, ty, tx) << 24;
    }
    kinfo[tid] = info;
  }
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
      *(u32x4*)&Ks[(ch / RCH) * KROW + (ch % RCH) * 8] = kreg[c];
      *(u32x4*)&Vs[(ch / RCH) * VROW + (ch % RCH) * 8] = vreg[c];
    }
  }
  __syncthreads();
  if (wave * 16 >= N) return;  // no barrier below this point

  // S^T = K Q^T for the 4 key blocks; keys past Nk start from -inf.
  f32x4 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[kb][r] = kb * 16 + g * 4 + r < Nk ? 0.f : -INFINITY;
#pragma unroll
    for (int dc = 0; dc < KCH; ++dc) {
      const u32x4 kf = *(const u32x4*)&Ks[(kb * 16 + l16) * KROW + dc * 32 + g * 8];
      s[kb] = E::mfma(kf, qf[dc], s[kb]);
    }
  }

  // Bias and mask (log2 units).  The region test is needed only when this
  // window straddles a shifted-region boundary.
  const float c2 = a.scale * kLog2e;
  const float mval = a.mask_value * kLog2e;
  int qtab = 0, qreg = 0;
  if constexpr (BIAS == ATTN_BIAS_TABLE) {
    const int qh = div_small(q_tok, inv_gw), qw = q_tok - qh * a.gw;
    qtab = (qh + a.gh - 1) * (2 * a.gw - 1) + qw + a.gw - 1;
  }
  if (regions) {
    int ty, tx;
    split(q_tok, ty, tx);
    qreg = win_region(a, pos, ty, tx);
  }
  // This lane's keys are kb*16 + g*4 + r: four consecutive kinfo entries.
  int ki[16];
  if (BIAS == ATTN_BIAS_TABLE || regions) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 v = *(const u32x4*)&kinfo[kb * 16 + g * 4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ki[kb * 4 + r] = (int)v[r];
    }
  }
  float y[16];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = min(kb * 16 + g * 4 + r, Nk - 1);
      float bias = 0.f;
      if constexpr (BIAS == ATTN_BIAS_TABLE) bias = tbl[qtab - (ki[kb * 4 + r] & 0xffffff)];
      if constexpr (BIAS == ATTN_BIAS_ADDITIVE)
        bias = load_elem<E>(a.badd, (int64_t)(b % a.badd_n) * a.badd_s0 + (int64_t)q_tok * a.badd_s1 + j) * kLog2e;
      if constexpr (MASKK == ATTN_MASK_ADDITIVE)
        bias += load_elem<E>(a.madd, (int64_t)(b % a.madd_n) * a.madd_s0 + (int64_t)q_tok * a.madd_s1 + j) * kLog2e;
      y[kb * 4 + r] = fmaf(s[kb][r], c2, bias);
    }
  if (regions) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((ki[e] >> 24) != qreg) y[e] += mval;
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
  u32x4 pf[2];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
    pf[kc] = u32x4{E::pack2(y[kc * 8 + 0], y[kc * 8 + 1]), E::pack2(y[kc * 8 + 2], y[kc * 8 + 3]),
                   E::pack2(y[kc * 8 + 4], y[kc * 8 + 5]), E::pack2(y[kc * 8 + 6], y[kc * 8 + 7])};

  // O^T += V^T P^T with transposing reads of the V tile.
  f32x4 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
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

  const float inv = __builtin_amdgcn_rcpf(sum_across_groups(ps));
  const int qi = wave * 16 + l16;
  if (qi < N) {
    const uint32_t off = row_off(qi, a.o_sn);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c0 = cb * 16 + g * 4;
      if (c0 < D) {
        const f32x4 v = o[cb] * inv;
        *(u32x2*)(op + (off + (uint32_t)c0)) = u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
      }
    }
  }
}

}  // namespace attn

#endif  // ATTN_WIN_H_
