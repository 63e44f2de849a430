// Half-precision attention kernel on gfx950 matrix cores.
//
// One workgroup = NW waves = a tile of BM = NW*NQB*16 queries of one
// (batch item, head).  Each wave owns NQB blocks of 16 queries and streams
// key/value tiles of 64 tokens through LDS (double buffered, 16-byte loads
// and stores, rows padded against bank conflicts).
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32:
//   A = K rows from LDS (lane l: key l%16, 8 head-dim elements (l/16)*8..),
//   B = Q^T kept in registers for the whole key loop,
//   C: lane l holds the scores of query l%16 for keys (l/16)*4 + r, r < 4.
// So every lane owns one query: the row max / row sum need only two
// cross-lane steps (v_permlane16_swap, v_permlane32_swap), the output
// rescale is one scalar per lane, and the probabilities are already laid out
// as the B operand of O^T += V^T P^T.  The A operand V^T is read straight
// from the row-major V tile with ds_read_b64_tr_b16 (16-lane transposing
// reads), with the key order of each 32-key chunk matching the score layout.
//
// The softmax runs in base 2 (exp2 of log2(e)-scaled logits) with a lazily
// updated row reference: the output is rescaled only when some row's
// maximum grew by more than 2^8, which keeps every probability <= 256 and
// skips almost every rescale after the first tiles.  This is the same
// softmax: any reference value gives the same normalised result.
//
// Relative position (SAM), fast form for 64-wide token grids: a key tile is
// exactly one grid row, so q.Rw[qw-kw+63] depends only on the key's place in
// the tile and is used as the initial accumulator of the QK^T MFMA chain
// (zero extra instructions per score), while q.Rh[qh-kh+63] is one scalar per
// query and tile, folded into the row offset.  Both come from small MFMA
// products of the query block with Rw / Rh in the prologue.
#ifndef ATTN_MFMA_H_
#define ATTN_MFMA_H_

#include "attn_device.h"

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));

#ifndef ATTN_MAX2
#define ATTN_MAX2 1  // joint cross-group maxima of a wave's two query blocks
#endif

// Word 3 of a buffer resource on gfx9-family chips: 32-bit data format,
// no swizzle.  With stride 0 the resource is "raw": an access at byte offset
// >= num_records returns zero and touches no memory.
constexpr int kBufferWord3 = 0x00020000;

// Raw buffer resource over [p, p + nrec bytes).  p and nrec must be the same
// in every lane of the wave (they are taken from the first active lane, so
// the resource lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t nrec) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0,
                                           (int)__builtin_amdgcn_readfirstlane(nrec), kBufferWord3);
}

// Tile geometry (MfmaCfg), the relative-position forms and the LDS byte
// counts are in attn_plan.h, shared with the host-side kernel choice.

// The lane index, recomputed where it is used: the asm is opaque to the
// compiler, so lane-constant values derived from it are not kept alive in
// registers across the key loop (which spilled two of them in the
// contraction form).
__device__ __forceinline__ int lane_id_here() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

__device__ __forceinline__ float max_across_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Row maxima of two values at once: on return every lane of `a` holds the
// maximum of a over the four 16-lane groups for its lane index l16, and
// likewise for `b`.  Seven instructions instead of twelve for two calls of
// max_across_groups.  v_permlane16_swap(x, y) exchanges the odd 16-lane rows
// of x with the even rows of y; v_permlane32_swap(x, y) rows 2-3 of x with
// rows 0-1 of y.
__device__ __forceinline__ void max_across_groups2(float& a, float& b) {
  // [a0, b0, a2, b2] and [a1, b1, a3, b3] -> [A01, B01, A23, B23]
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const float m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  // [A01, B01, A01, B01] and [A23, B23, A23, B23] -> [A, B, A, B]
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  const float n = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  // [A, A, A, A] and [B, B, B, B]
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(n), __float_as_uint(n), false, false);
  a = __uint_as_float(t[0]);
  b = __uint_as_float(t[1]);
}

__device__ __forceinline__ float sum_across_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-lane transposing LDS read: lane j of a 16-lane group receives element
// j%4 of the 4-element chunks addressed by lanes j/4, j/4+4, j/4+8, j/4+12.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const s16x4 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// WPE: waves per SIMD the register allocation targets (2 lets the softmax of
// one wave overlap the matrix products of another).
#ifndef ATTN_WPE_ATTR
#define ATTN_WPE_ATTR 1
#endif
#if ATTN_WPE_ATTR
#define ATTN_WAVES_PER_EU(n) __attribute__((amdgpu_waves_per_eu(n, n)))
#else
#define ATTN_WAVES_PER_EU(n)
#endif
// IMG: built with the image-layout addressing (the batched-layout instance
// leaves it out, which keeps the key loop within fewer registers).
template <class E, int D, int NW, int NQB, int BIAS, bool MASK, int RMODE, int WPE, bool IMG,
          bool F8 = false>
__global__ __launch_bounds__(NW * 64) ATTN_WAVES_PER_EU(WPE) void attn_fwd_mfma(AttnArgs a) {
  // F8: q, k, v are E4M3 codes, loaded as 8-byte pieces per 8 elements and
  // widened exactly to E (Q in registers, K/V on their way into LDS); the q
  // and k scales ride in a.scale, the v scale is applied with the row-sum
  // division.  Built for the forms without relative position.
  static_assert(!F8 || (BIAS != ATTN_BIAS_RELPOS && (RMODE == kRelTables || RMODE == kTwoTiles)),
                "8-bit inputs are built for the forms without relative position");
  constexpr int IES = F8 ? 1 : 2;                     // bytes of a q, k or v element
  using LdT = std::conditional_t<F8, u32x2, u32x4>;  // one 8-element chunk as loaded
  constexpr bool RFAST = RMODE == kRelRow64;
  constexpr bool RAUG = RMODE == kRelAug;
  constexpr bool PP = NW == 8 && RMODE != kTwoTiles;  // ping-pong schedule of two wave groups
  static_assert(!PP || !RAUG, "the ping-pong schedule is not built for the augmented contraction");
  static_assert(!(PP && IMG), "the ping-pong form is launched for the batched layout only");
  if constexpr (!IMG) a.image = 0;
  using C = MfmaCfg<D, NW, NQB, RAUG>;
  constexpr int NT = C::NT, BM = C::BM, BN = C::BN, KCH = C::KCH, KCHT = C::KCHT, DK = C::DK,
                CB = C::CB, DV = C::DV, KROW = C::KROW, VROW = C::VROW, RCH = C::RCH,
                NCH = C::NCH, CPT = C::CPT;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* Ks = (uint16_t*)lds;          // [2][BN][KROW]
  uint16_t* Vs = Ks + 2 * C::K_ELEMS;     // [2][BN][VROW]

  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int l16 = lane & 15, g = lane >> 4;
  int bid = xcd_logical_id(__builtin_amdgcn_workgroup_id_x(), a.n_blocks);
  const int qt_div = fdiv(bid, a.fd_qt);
  const int qt = bid - qt_div * a.n_qtiles;
  const int b = fdiv(qt_div, a.fd_h);
  const int h = qt_div - b * a.H;
  // The two-tile form in the batched layout walks tpw consecutive query
  // tiles per workgroup (q0 advances by BM after each), except at d = 64,
  // where its output staging would cost a resident workgroup per CU.
  constexpr bool kPersist = RMODE == kTwoTiles && !IMG && two_tile_persists<D>();
  const int q0 = qt * (kPersist ? max(a.tpw, 1) : 1) * BM;
  const int wq0 = wave * NQB * 16;  // first query row of this wave inside the tile

  // Query fragments (B operand of S^T = K Q^T): lane holds Q[q][dc*32 + g*8 .. +7].
  u32x4 qf[NQB][KCHT];
  const char* qbase = (const char*)a.q + IES * tok_base(a, a.q_sb, a.q_sh, b, h);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qi = min(q0 + wq0 + qb * 16 + l16, a.Nq - 1);
    const uint32_t off = tok_row(a, a.q_sn, b, qi);
#pragma unroll
    for (int dc = 0; dc < KCH; ++dc) {
      const int d0 = dc * 32 + g * 8;
      // (a padding token of the image layout is a zero query)
      if constexpr (F8) {
        // Loaded from an address that is always valid and then selected, so
        // the loads of all fragments are in flight together (a load inside
        // the condition would be waited for before its conversion).
        const bool ok = d0 < D && off != kPadTok;
        const u32x4 wq = widen_e4m3<E>(*(const u32x2*)(qbase + (ok ? off + d0 : 0)));
        qf[qb][dc] = ok ? wq : u32x4{0, 0, 0, 0};
      } else
        qf[qb][dc] = d0 < D && off != kPadTok ? *(const u32x4*)(qbase + 2 * (off + d0)) : u32x4{0, 0, 0, 0};
    }
  }

  // Tile loaders: CPT 16-byte chunks of K and of V per thread, through
  // buffer resources.  Batched layout: the resource of tile t starts at key
  // t*BN and ends with the last byte of key Nk-1, so a chunk's byte offset is
  // the same in every tile and chunks of keys past Nk read as zero without a
  // memory access.  Image layout: per-key offsets through the window map,
  // with keys past Nk clamped to Nk-1.  Either way those keys' scores are
  // set to -inf before the softmax.
  const char* kbase = (const char*)a.k + IES * tok_base(a, a.k_sb, a.k_sh, b, h);
  const char* vbase = (const char*)a.v + IES * tok_base(a, a.v_sb, a.v_sh, b, h);
  LdT kreg[CPT], vreg[CPT];
  auto crow = [&](int c) { const int ch = tid + c * NT; return ch < NCH ? ch / RCH : (1 << 29); };
  auto ccol = [&](int c) { return ((tid + c * NT) % RCH) * 8; };
  uint32_t koff[CPT], voff[CPT];  // batched layout: chunk byte offsets inside a tile
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int r = crow(c);
    const int64_t ko = (int64_t)r * a.k_sn + ccol(c), vo = (int64_t)r * a.v_sn + ccol(c);
    koff[c] = r < BN && IES * ko < 0xFFFFFFF0ll ? (uint32_t)(IES * ko) : 0xFFFFFFF0u;
    voff[c] = r < BN && IES * vo < 0xFFFFFFF0ll ? (uint32_t)(IES * vo) : 0xFFFFFFF0u;
  }
  // Image layout: key j's window-map pixel (kPadTok for padding), filled
  // once below; the tile loads after the first barrier read it instead of
  // evaluating the map per chunk and tile.
  uint32_t* kpix = (uint32_t*)(lds + mfma_lds_bytes<D, NW, NQB, RMODE>(a) - img_key_bytes(a));
  if constexpr (IMG) {
    for (int j = tid; j < a.Nk; j += NT) kpix[j] = tok_row(a, 1, b, j);
  }
  auto buf_load = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off) -> LdT {
    if constexpr (F8) return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  };
  auto load_rows = [&](const char* base, int64_t sn, const uint32_t* off, int t, LdT* reg,
                       bool direct = false) {
    if (!a.image) {
      const int64_t k0 = (int64_t)t * BN;
      const uint32_t nrec = (uint32_t)(IES * ((a.Nk - 1 - k0) * sn + D));
      const auto rs = buffer_rsrc(base + IES * k0 * sn, nrec);
#pragma unroll
      for (int c = 0; c < CPT; ++c) reg[c] = buf_load(rs, off[c]);
    } else {
      // Padding tokens read at a byte offset past the resource's range,
      // which gives zero (in-slice offsets stay below 2^30 bytes).
      const auto rs = buffer_rsrc(base, 0xFFFFFFF0u);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int key = min(t * BN + min(crow(c), BN - 1), a.Nk - 1);
        uint32_t r;
        if (direct) {
          r = tok_row(a, sn, b, key);  // before the first barrier: kpix is not ready
        } else {
          const uint32_t px = kpix[key];
          r = px == kPadTok ? kPadTok : px * (uint32_t)sn;
        }
        reg[c] = buf_load(rs, r == kPadTok ? 0xFFFFFFF0u : IES * (r + (uint32_t)ccol(c)));
      }
    }
  };
  auto load_k = [&](int t) { load_rows(kbase, a.k_sn, koff, t, kreg); };
  auto load_v = [&](int t) { load_rows(vbase, a.v_sn, voff, t, vreg); };
  auto widen = [&](LdT x) -> u32x4 {
    if constexpr (F8) return widen_e4m3<E>(x);
    else return x;
  };
  auto store_k_from = [&](int st, int t, const LdT* src) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (crow(c) < BN) *(u32x4*)&Ks[st * C::K_ELEMS + crow(c) * KROW + ccol(c)] = widen(src[c]);
    if constexpr (RAUG) {
      // One-hot chunk of key row `row`: ones at columns kh and gh + kw.
      for (int i = tid; i < BN * 4; i += NT) {
        const int row = i >> 2, cq = (i & 3) * 8;
        const int j = t * BN + row;
        // (j + 0.5) / gw is within 0.004 of j / gw and gw <= 31, so the
        // truncation is exact for j < 16384.
        const int kh = (int)(((float)j + 0.5f) / (float)a.gw), kw = j - kh * a.gw;
        uint32_t w4[4] = {0, 0, 0, 0};
        const uint32_t one = E::one_bits();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int col = cq + e;
          if (j < a.Nk && (col == kh || col == a.gh + kw)) w4[e >> 1] |= one << ((e & 1) * 16);
        }
        *(u32x4*)&Ks[st * C::K_ELEMS + row * KROW + KCH * 32 + cq] = u32x4{w4[0], w4[1], w4[2], w4[3]};
      }
    }
  };
  auto store_v_from = [&](int st, const LdT* src) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (crow(c) < BN) *(u32x4*)&Vs[st * C::V_ELEMS + crow(c) * VROW + ccol(c)] = widen(src[c]);
  };
  auto store_k = [&](int st, int t) { store_k_from(st, t, kreg); };
  auto store_v = [&](int st) { store_v_from(st, vreg); };

  // Augmented relative position: A fragments of the stacked table [Rh; Rw]
  // ((2gh-1) + (2gw-1) <= 62 rows, so four 16-row blocks), issued before the
  // K/V tile loads so that the prologue waits for these and Q only.
  constexpr int RFB = RAUG ? 4 : 1;
  u32x4 rfrag[RFB][RAUG ? KCH : 1];
  if constexpr (RAUG) {
    const int nh = 2 * a.gh - 1, nrows = nh + 2 * a.gw - 1;
#pragma unroll
    for (int mb = 0; mb < RFB; ++mb) {
      const int m = mb * 16 + l16;
      const uint16_t* row = m < nh ? (const uint16_t*)a.rh + (int64_t)m * D
                                   : (const uint16_t*)a.rw + (int64_t)(m < nrows ? m - nh : 0) * D;
#pragma unroll
      for (int dc = 0; dc < KCH; ++dc) {
        const int d0 = dc * 32 + g * 8;
        rfrag[mb][dc] = m < nrows && d0 < D ? *(const u32x4*)(row + d0) : u32x4{0, 0, 0, 0};
      }
    }
  }

  // Row form (64-wide grids): A fragments of all 127 Rw rows and of the
  // first 64 Rh rows this wave needs.  A wave's 32 queries start at a
  // multiple of 32 and Nq = 64 gh, so they lie in one grid row qh_w (clamped
  // queries past Nq fall in the last row, as does Nq - 1) and share Rh rows.
  constexpr int RWB = RFAST ? 8 : 1, RHB = RFAST ? 4 : 1, RKC = RFAST ? KCH : 1;
  u32x4 wfrag[RWB][RKC], hfrag[RHB][RKC];
  const int qh_w = min(q0 + wq0, a.Nq - 1) >> 6;
  auto load_hfrag = [&](int mb0) {
#pragma unroll
    for (int mb = 0; mb < RHB; ++mb) {
      const int kh_row = (mb0 + mb) * 16 + l16;
      const uint16_t* row = (const uint16_t*)a.rh + (int64_t)(kh_row < a.gh ? qh_w + a.gh - 1 - kh_row : 0) * D;
#pragma unroll
      for (int dc = 0; dc < RKC; ++dc) {
        const int d0 = dc * 32 + g * 8;
        hfrag[mb][dc] = kh_row < a.gh && d0 < D ? *(const u32x4*)(row + d0) : u32x4{0, 0, 0, 0};
      }
    }
  };
  if constexpr (RFAST) {
#pragma unroll
    for (int mb = 0; mb < RWB; ++mb) {
      const int m_row = mb * 16 + l16;
#pragma unroll
      for (int dc = 0; dc < RKC; ++dc) {
        const int d0 = dc * 32 + g * 8;
        wfrag[mb][dc] = m_row < 127 && d0 < D ? *(const u32x4*)((const uint16_t*)a.rw + (int64_t)m_row * D + d0)
                                              : u32x4{0, 0, 0, 0};
      }
    }
    load_hfrag(0);
  }

  // The first K/V tile is in flight while the bias prologue runs.  When the
  // keys span exactly two tiles, the second one is loaded with it: both
  // stages are then filled once and no load waits between the tiles.
  load_rows(kbase, a.k_sn, koff, 0, kreg, true);
  load_rows(vbase, a.v_sn, voff, 0, vreg, true);
  constexpr bool TWO = RMODE == kTwoTiles;
  static_assert(!TWO || (!PP && BIAS == ATTN_BIAS_NONE && !MASK), "two-tile form: no bias, no mask");
  LdT kreg1[TWO ? CPT : 1], vreg1[TWO ? CPT : 1];
  if constexpr (TWO) {
    load_rows(kbase, a.k_sn, koff, 1, kreg1, true);
    load_rows(vbase, a.v_sn, voff, 1, vreg1, true);
  }

  BiasCtx bc;
  QInfo qinf[NQB];
  f32x4 sinit[4][NQB];
  const float* relh_lds = nullptr;
  if constexpr (RFAST) {
    // Relative position for a 64-wide grid (tile t = grid row t).
    float* relh_tab = (float*)(lds + C::BASE_BYTES);  // [gh][BM], log2 units
    float* gscr = (float*)lds + wave * 16 * C::GROW;   // per-wave scratch, overlays K/V
    const float inv_scale = 1.f / a.scale;
    // relh[i][kh] = Rh[qh + gh - 1 - kh] . q_i, as C[kh][i] of an MFMA product.
    for (int mb0 = 0; mb0 * 16 < a.gh; mb0 += RHB) {
      if (mb0 > 0) load_hfrag(mb0);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int il0 = wq0 + qb * 16;
#pragma unroll
        for (int mb = 0; mb < RHB; ++mb) {
          if ((mb0 + mb) * 16 >= a.gh) break;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < KCH; ++dc) acc = E::mfma(hfrag[mb][dc], qf[qb][dc], acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kh = (mb0 + mb) * 16 + g * 4 + r;
            if (kh < a.gh) relh_tab[kh * BM + il0 + l16] = acc[r] * kLog2e;
          }
        }
      }
    }
    // G[m][i] = Rw[m] . q_i for every table row m, then the per-lane gather
    // relw[i][kw] = G[qw_i + 63 - kw][i] for this lane's 16 keys.
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int mb = 0; mb < RWB; ++mb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < KCH; ++dc) acc = E::mfma(wfrag[mb][dc], qf[qb][dc], acc);
        *(f32x4*)&gscr[l16 * C::GROW + mb * 16 + g * 4] = acc;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int qw = min(q0 + wq0 + qb * 16 + l16, a.Nq - 1) & 63;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sinit[kb][qb][r] = gscr[l16 * C::GROW + qw + 63 - (kb * 16 + g * 4 + r)] * inv_scale;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    relh_lds = relh_tab;
  } else if constexpr (RAUG) {
    // Relative position folded into the contraction: the extra Q chunk holds
    // relh[i][0..gh) and relw[i][0..gw) divided by the scale (the K tile's
    // extra chunk holds one-hots at kh and gh + kw), so QK^T directly gives
    // q.k + (relh + relw) / scale.  G = [Rh; Rw] Q^T comes from the matrix
    // cores and is gathered per lane through this wave's scratch rows.
    float* gscr = (float*)lds + wave * 16 * kAugGrow;  // overlays the K/V tiles
    const int nh = 2 * a.gh - 1, nrows = nh + 2 * a.gw - 1;
    const float inv_scale = 1.f / a.scale;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qi = min(q0 + wq0 + qb * 16 + l16, a.Nq - 1);
      const int qh = fdiv(qi, a.fd_gw), qw = qi - qh * a.gw;
#pragma unroll
      for (int mb = 0; mb < RFB; ++mb) {
        if (mb * 16 >= nrows) break;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < KCH; ++dc) acc = E::mfma(rfrag[mb][dc], qf[qb][dc], acc);
        *(f32x4*)&gscr[l16 * kAugGrow + mb * 16 + g * 4] = acc;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // Extension column k = g*8 + e: relh[kh = k] (stacked row qh - kh + gh - 1)
      // or relw[kw = k - gh] (stacked row nh + qw - kw + gw - 1).
      float ext[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = g * 8 + e, kw = k - a.gh;
        const bool in = k < a.gh + a.gw;
        const int m = !in ? 0 : k < a.gh ? qh - k + a.gh - 1 : nh + qw - kw + a.gw - 1;
        const float gv = gscr[l16 * kAugGrow + m] * inv_scale;
        ext[e] = in ? gv : 0.f;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      qf[qb][KCH] = u32x4{E::pack2(ext[0], ext[1]), E::pack2(ext[2], ext[3]), E::pack2(ext[4], ext[5]),
                          E::pack2(ext[6], ext[7])};
    }
  } else {
    setup_bias<E, BIAS, MASK, BM, NT, false>(a, lds + C::KV_BYTES, b, h, q0, bc);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int il = wq0 + qb * 16 + l16;
      qinf[qb] = make_qinfo<BIAS, MASK>(a, b, min(q0 + il, a.Nq - 1), il);
    }
    if constexpr (BIAS == ATTN_BIAS_RELPOS && !RAUG) {
      // relh[kh][i] = q_i . Rh[rel_row(qh_i, kh)] and relw[kw][i] likewise
      // (kh, kw on the key grid; equal grids: Rh[qh_i - kh + gh - 1]):
      // G = R Q^T on the matrix cores for every table row, then a per-lane
      // gather through this wave's scratch rows.
      const int grow = relpos_grow(a);
      float* gscr = (float*)(lds + mfma_lds_bytes<D, NW, NQB>(a) - img_key_bytes(a)) - (NW - wave) * 16 * grow;
      float* relh = (float*)bc.relh;
      float* relw = (float*)bc.relw;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int il = wq0 + qb * 16 + l16;
        const int qi = min(q0 + il, a.Nq - 1);
        const int qh = fdiv(qi, a.fd_gw), qw = qi - qh * a.gw;
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const int gg = part == 0 ? a.gh : a.gw;    // query positions on this axis
          const int kg = part == 0 ? a.kgh : a.kgw;  // key positions
          const int nrow = 2 * (gg > kg ? gg : kg) - 1;  // rows the grids need
          const int nsrc = part == 0 ? a.rh_rows : a.rw_rows;  // rows stored
          const uint16_t* tab = (const uint16_t*)(part == 0 ? a.rh : a.rw);
          for (int mb = 0; mb * 16 < nsrc; ++mb) {
            const int m_row = mb * 16 + l16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < KCH; ++dc) {
              const int d0 = dc * 32 + g * 8;
              u32x4 af = {0, 0, 0, 0};
              if (m_row < nsrc && d0 < D) af = *(const u32x4*)(tab + (int64_t)m_row * D + d0);
              acc = E::mfma(af, qf[qb][dc], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) gscr[l16 * grow + mb * 16 + g * 4 + r] = acc[r];
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int qc = part == 0 ? qh : qw;
          float* dst = part == 0 ? relh : relw;
          // A table stored at another length is resized here: the product
          // with q is linear, so interpolating G between stored rows equals
          // the product with the interpolated row.
          for (int kk = g; kk < kg; kk += 4) {
            int i0, i1;
            float f;
            resized_row(rel_row(qc, kk, gg, kg), nsrc, nrow, i0, i1, f);
            const float g0 = gscr[l16 * grow + i0];
            dst[kk * BM + il] = fmaf(f, gscr[l16 * grow + i1] - g0, g0) * kLog2e;
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
    }
  }

  const float c2 = a.scale * kLog2e;  // logits in log2 units = c2 * (q.k)
  const int ntiles = (a.Nk + BN - 1) / BN;
  // Transposing V reads: this lane addresses key row (l16 / 4) of its group's
  // 4-key slice and channel block 4 * (l16 % 4).
  const int vt_row = g * 4 + (l16 >> 2), vt_col = 4 * (l16 & 3);
  // When D is a multiple of 16, the last 16-row block of V^T holds only the
  // ones row (row D) and zeros: its fragment is a constant (one in every
  // element of the lanes of row 0), taken from registers instead of LDS.
  constexpr bool kOnesBlock = C::ONES && D % 16 == 0;
  const uint32_t one2 = l16 == 0 ? (uint32_t)E::one_bits() * 0x10001u : 0u;
  const u32x4 ones_frag = u32x4{one2, one2, one2, one2};
  // S^T = K Q^T for one key tile.  All K fragments are read first, so the
  // LDS latency is paid once per tile.  The first product of each chain
  // takes its addend directly: zero, or the row-form relative-position term.
  // nkb: key blocks of 16 holding keys below Nk (4 except in a ragged last
  // tile, whose empty blocks are skipped: their scores are masked anyway).
  // The contraction form holds one more K chunk and targets one more wave
  // per SIMD than the other forms: it reads the K fragments of two key blocks
  // at a time and the V^T fragments after the softmax, which keeps its peak
  // register count within the smaller budget.
  constexpr bool kLean = RAUG;
  auto qk = [&](const uint16_t* Kt, f32x4 (&s)[4][NQB], int nkb = 4) {
    constexpr int KBB = kLean ? 2 : 4;  // key blocks whose fragments are read together
#pragma unroll
    for (int kb0 = 0; kb0 < 4; kb0 += KBB) {
    u32x4 kf[KCHT][4];
#pragma unroll
    for (int dc = 0; dc < KCHT; ++dc)
#pragma unroll
      for (int kb = kb0; kb < kb0 + KBB; ++kb)
        if (kb < nkb) kf[dc][kb] = *(const u32x4*)&Kt[(kb * 16 + l16) * KROW + dc * 32 + g * 8];
#pragma unroll
    for (int dc = 0; dc < KCHT; ++dc) {
#pragma unroll
      for (int kb = kb0; kb < kb0 + KBB; ++kb) {
        if (kb >= nkb) continue;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          f32x4 c = s[kb][qb];
          if (dc == 0) {
            if constexpr (RFAST) c = sinit[kb][qb];
            else c = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          s[kb][qb] = E::mfma(kf[dc][kb], qf[qb][dc], c);
        }
      }
    }
    }
  };

  f32x4 o[CB][NQB];
  float m[NQB], l[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[cb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One key tile t: row maxima and the lazy rescale of the output, then the
  // exponentials and O^T += V^T P^T.  The V^T fragments are read from LDS
  // before the softmax so their latency hides behind it (after it in the
  // contraction form, for the register budget).  Keys past Nk can
  // only occur in the last tile (never with the 64-wide row form).
  f32x4 s_cur[4][NQB];
  const bool ragged = (a.Nk % BN) != 0;
  auto tile = [&](int t, auto last) {
    constexpr bool LAST = decltype(last)::value && !RFAST;
    const int k0 = t * BN;
    // Keys 32..63 of a ragged last tile may all lie past Nk, and so may
    // whole 16-key blocks: those take no part in the softmax (their
    // probabilities are zero).
    const int nkc = LAST && k0 + 32 >= a.Nk ? 1 : 2;
    constexpr bool kGenericBias = RMODE == kRelTables && (BIAS != ATTN_BIAS_NONE || MASK);
    constexpr bool SKIP = LAST && !kGenericBias;  // (per-score bias forms keep the full tile)
    const int nkbt = SKIP ? min(4, (a.Nk - k0 + 15) / 16) : 4;
    const uint16_t* Vt = Vs + (t & 1) * C::V_ELEMS;
    u32x4 vf[2][CB];
    auto read_vf = [&]() {
      int vr = vt_row, vc = vt_col;
      if constexpr (kLean) {
        const int ln = lane_id_here();
        vr = (ln >> 4) * 4 + ((ln & 15) >> 2);
        vc = 4 * (ln & 3);
      }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (kc >= nkc) continue;
        if (kOnesBlock && cb == CB - 1) {
          vf[kc][cb] = ones_frag;
          continue;
        }
        const uint16_t* vp = Vt + (kc * 32 + vr) * VROW + cb * 16 + vc;
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 16 * VROW);
        vf[kc][cb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    };
    if constexpr (!kLean) read_vf();
    const float cy = kGenericBias ? 1.f : c2;
    float y[NQB][16];
    float nb[NQB];
    u32x4 pf[NQB][2];
    // p = 2^(y*cy + nb), rounded to the element type as the B operand of PV.
    auto exp_pack = [&](int qb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float& e = y[qb][kb * 4 + r];
          if (!SKIP || kb == 0 || kb < nkbt) e = __builtin_amdgcn_exp2f(fmaf(e, cy, nb[qb]));
          else e = 0.f;
        }
      if constexpr (!C::ONES) {
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ps += y[qb][i];
        l[qb] += ps;
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        if (!SKIP || kc < nkc)
        pf[qb][kc] = u32x4{E::pack2(y[qb][kc * 8 + 0], y[qb][kc * 8 + 1]),
                           E::pack2(y[qb][kc * 8 + 2], y[qb][kc * 8 + 3]),
                           E::pack2(y[qb][kc * 8 + 4], y[qb][kc * 8 + 5]),
                           E::pack2(y[qb][kc * 8 + 6], y[qb][kc * 8 + 7])};
    };
    float hq[NQB], mq[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      hq[qb] = 0.f;
      if constexpr (RFAST) hq[qb] = relh_lds[t * BM + wq0 + qb * 16 + l16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = s_cur[kb][qb][r];
          if constexpr (kGenericBias) {
            const int kj = k0 + kb * 16 + g * 4 + r;
            v = fmaf(v, c2, bias_log2<E, BIAS, MASK, BM>(a, bc, qinf[qb], b, min(kj, a.Nk - 1)));
          }
          y[qb][kb * 4 + r] = v;
        }
      if (LAST && ragged) {
        // Keys past Nk leave the softmax.
        const int lim = a.Nk - k0 - g * 4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb * 16 + r >= lim) y[qb][kb * 4 + r] = -INFINITY;
      }
      float mx;
      if constexpr (SKIP) {
        mx = fmaxf(fmaxf(y[qb][0], y[qb][1]), fmaxf(y[qb][2], y[qb][3]));
#pragma unroll
        for (int kb = 1; kb < 4; ++kb)
          if (kb < nkbt)
            mx = fmaxf(mx, fmaxf(fmaxf(y[qb][kb * 4], y[qb][kb * 4 + 1]), fmaxf(y[qb][kb * 4 + 2], y[qb][kb * 4 + 3])));
      } else {
        mx = fmaxf(fmaxf(y[qb][0], y[qb][1]), y[qb][2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, y[qb][i]), y[qb][i + 1]);
        mx = fmaxf(mx, y[qb][15]);
      }
      mq[qb] = mx;
    }
    if constexpr (NQB == 2 && ATTN_MAX2 && !kLean) {
      max_across_groups2(mq[0], mq[1]);
    } else {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) mq[qb] = max_across_groups(mq[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float hh = hq[qb];
      const float mt = fmaf(mq[qb], cy, hh);  // tile row maximum, log2 units
      if (__builtin_amdgcn_ballot_w64(mt > m[qb] + 8.f)) {
        const float mn = fmaxf(m[qb], mt);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[qb] - mn);
        m[qb] = mn;
        if constexpr (!C::ONES) l[qb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb][qb] *= alpha;
      }
      nb[qb] = hh - (m[qb] == -INFINITY ? 0.f : m[qb]);
      exp_pack(qb);
    }
    // O^T += V^T P^T.
    if constexpr (kLean) {
      __builtin_amdgcn_sched_barrier(0);
      read_vf();
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (kc >= nkc) continue;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) o[cb][qb] = E::mfma(vf[kc][cb], pf[qb][kc], o[cb][qb]);
      }
  };

  // Ping-pong schedule (8-wave workgroups): the softmax of tile t producing
  // the packed probabilities, and the matrix phase PV(t-1) + QK(t).
  u32x4 pp_p[NQB][2];
  auto softmax_pp = [&](int t, auto last) {
    constexpr bool LAST = decltype(last)::value && !RFAST;
    const int k0 = t * BN;
    constexpr bool kGenericBias = RMODE == kRelTables && (BIAS != ATTN_BIAS_NONE || MASK);
    const float cy = kGenericBias ? 1.f : c2;
    float yy[NQB][16], hq[NQB], mq[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float* y = yy[qb];
      hq[qb] = 0.f;
      if constexpr (RFAST) hq[qb] = relh_lds[t * BM + wq0 + qb * 16 + l16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = s_cur[kb][qb][r];
          if constexpr (kGenericBias) {
            const int kj = k0 + kb * 16 + g * 4 + r;
            v = fmaf(v, c2, bias_log2<E, BIAS, MASK, BM>(a, bc, qinf[qb], b, min(kj, a.Nk - 1)));
          }
          y[kb * 4 + r] = v;
        }
      if (LAST && ragged) {
        const int lim = a.Nk - k0 - g * 4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb * 16 + r >= lim) y[kb * 4 + r] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(y[0], y[1]), y[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, y[i]), y[i + 1]);
      mq[qb] = fmaxf(mx, y[15]);
    }
    if constexpr (NQB == 2 && ATTN_MAX2) {
      max_across_groups2(mq[0], mq[1]);
    } else {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) mq[qb] = max_across_groups(mq[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float* y = yy[qb];
      const float hh = hq[qb];
      const float mt = fmaf(mq[qb], cy, hh);
      if (__builtin_amdgcn_ballot_w64(mt > m[qb] + 8.f)) {
        const float mn = fmaxf(m[qb], mt);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[qb] - mn);
        m[qb] = mn;
        if constexpr (!C::ONES) l[qb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb][qb] *= alpha;
      }
      const float nb = hh - (m[qb] == -INFINITY ? 0.f : m[qb]);
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = __builtin_amdgcn_exp2f(fmaf(y[i], cy, nb));
      if constexpr (!C::ONES) {
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ps += y[i];
        l[qb] += ps;
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        pp_p[qb][kc] = u32x4{E::pack2(y[kc * 8 + 0], y[kc * 8 + 1]), E::pack2(y[kc * 8 + 2], y[kc * 8 + 3]),
                             E::pack2(y[kc * 8 + 4], y[kc * 8 + 5]), E::pack2(y[kc * 8 + 6], y[kc * 8 + 7])};
    }
  };
  auto pv_pp = [&](int t) {
    const uint16_t* Vt = Vs + (t & 1) * C::V_ELEMS;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      u32x4 vf[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (kOnesBlock && cb == CB - 1) {
          vf[cb] = ones_frag;
          continue;
        }
        const uint16_t* vp = Vt + (kc * 32 + vt_row) * VROW + cb * 16 + vt_col;
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 16 * VROW);
        vf[cb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) o[cb][qb] = E::mfma(vf[cb], pp_p[qb][kc], o[cb][qb]);
    }
  };

  __syncthreads();  // prologue scratch (overlaying the K/V tiles) is free now
  // Padding columns of the K and V tiles are never loaded: zero them once.
  // Column D of V is set to 1, so row D of O^T accumulates the row sum of
  // the (rounded) probabilities on the matrix cores.
  if constexpr (KCH * 32 > D) {
    constexpr int P = KCH * 32 - D;
    for (int i = tid; i < 2 * BN * P; i += NT) {
      const int row = i / P, col = D + i % P;
      Ks[row * KROW + col] = 0;
    }
  }
  if constexpr (DV > D) {
    for (int i = tid; i < 2 * BN * (DV - D); i += NT) {
      const int row = i / (DV - D), col = D + i % (DV - D);
      Vs[row * VROW + col] = (C::ONES && col == D) ? E::one_bits() : 0;
    }
  }

  if constexpr (PP) {
    // Two groups of four waves (one wave of each per SIMD) alternate between
    // a matrix phase, PV(t-1) + QK(t), and a softmax phase, separated by
    // workgroup barriers; group B runs one phase behind group A, so while
    // one wave of a SIMD keeps the matrix cores busy the other one runs its
    // exponentials.  Tile t's K and tile t-1's V are read during phases 2t
    // and 2t+1; K(t+1) and V(t) are written into the other stages during
    // phase 2t+1 (by group A after its softmax, by group B after its matrix
    // phase), which is the last use of those stages' previous contents.
    const bool grp_b = wave >= NW / 2;
    // V(0) stays in registers (loaded before the prologue) until phase 1.
    store_k(0, 0);
    if (ntiles > 1) load_k(1);
    auto store_next = [&](int t) {
      if (t + 1 < ntiles) store_k((t + 1) & 1, t + 1);
      store_v(t & 1);
      if (t + 2 < ntiles) load_k(t + 2);
      if (t + 1 < ntiles) load_v(t + 1);
    };
    __syncthreads();
    if (grp_b) __syncthreads();
    auto iter = [&](int t, auto last) {
      __builtin_amdgcn_s_setprio(1);
      if (t > 0) pv_pp(t - 1);
      qk(Ks + (t & 1) * C::K_ELEMS, s_cur);
      __builtin_amdgcn_s_setprio(0);
      if (grp_b) store_next(t);
      __syncthreads();
      softmax_pp(t, last);
      if (!grp_b) store_next(t);
      __syncthreads();
    };
    for (int t = 0; t + 1 < ntiles; ++t) iter(t, std::false_type{});
    iter(ntiles - 1, std::true_type{});
    pv_pp(ntiles - 1);
    if (!grp_b) __syncthreads();
  } else if constexpr (TWO) {
  store_k(0, 0);
  store_v(0);
  store_k_from(1, 1, kreg1);
  store_v_from(1, vreg1);
  __syncthreads();
  if constexpr (kPersist) {
    // The workgroup's query tiles in turn against the staged K and V: no
    // workgroup barrier in the loop (each wave stages its own output rows
    // in a region of its own).
    const int q_end = min(a.Nq, q0 + max(a.tpw, 1) * BM);
    int qc = q0;  // the current tile's first query
    uint16_t* obase = (uint16_t*)a.o + tok_base(a, a.o_sb, a.o_sh, b, h);
    const bool staged = D % 8 == 0 && a.o_sn == D && ((a.o_sb | a.o_sh) & 7) == 0;
    uint16_t* stage = (uint16_t*)(lds + ((mfma_lds_bytes<D, NW, NQB, RMODE>(a) + 15) & ~(size_t)15)) +
                      wave * (NQB * 16 * D);
    constexpr int PLB = D / 16, PLG = (D % 16) / 4, PLR = D % 4;
    // The Q fragments of the tile starting at query qs, as in the prologue.
    auto load_qf = [&](int qs) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qi = min(qs + wq0 + qb * 16 + l16, a.Nq - 1);
        const uint32_t off = tok_row(a, a.q_sn, b, qi);
#pragma unroll
        for (int dc = 0; dc < KCH; ++dc) {
          const int d0 = dc * 32 + g * 8;
          // (a padding token of the image layout is a zero query)
          if constexpr (F8) {
            // Loaded from an address that is always valid and then selected,
            // so the loads of all fragments are in flight together (a load
            // inside the condition would be waited for before its conversion).
            const bool ok = d0 < D && off != kPadTok;
            const u32x4 wq = widen_e4m3<E>(*(const u32x2*)(qbase + (ok ? off + d0 : 0)));
            qf[qb][dc] = ok ? wq : u32x4{0, 0, 0, 0};
          } else
            qf[qb][dc] = d0 < D && off != kPadTok ? *(const u32x4*)(qbase + 2 * (off + d0)) : u32x4{0, 0, 0, 0};
        }
      }
    };
    while (true) {
      const int qn = qc + BM;
      const bool more = qn < q_end;  // (a wave with no row below Nq is in the last tile)
      if (qc + wq0 < a.Nq) {
        qk(Ks, s_cur);
        tile(0, std::false_type{});
        qk(Ks + C::K_ELEMS, s_cur, min(4, (a.Nk - BN + 15) / 16));
        if (more) load_qf(qn);  // Q is not read again in this tile: the next tile's rows in flight
        tile(1, std::true_type{});
        // Normalise by the row sum and store this tile's rows of the wave.
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float lsum;
          if constexpr (C::ONES) lsum = __shfl(o[PLB < CB ? PLB : 0][qb][PLR], PLG * 16 + l16);
          else lsum = sum_across_groups(l[qb]);
          const float inv = (F8 ? a.v_descale : 1.f) / lsum;
          const int qi = qc + wq0 + qb * 16 + l16;
          if (a.lse && g == 0 && qi < a.Nq)
            a.lse[((int64_t)b * a.H + h) * a.Nq + qi] = (m[qb] + __builtin_amdgcn_logf(lsum)) * kLn2;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const int c0 = cb * 16 + g * 4;
            if (c0 < D) {
              const f32x4 v = o[cb][qb] * inv;
              const u32x2 packed = {E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
              if (staged) *(u32x2*)(stage + (qb * 16 + l16) * D + c0) = packed;
              else if (qi < a.Nq)
                __builtin_nontemporal_store(packed, (u32x2*)(obase + tok_row(a, a.o_sn, b, qi) + c0));
            }
          }
        }
        if (staged) {
          // The wave's NQB*16 rows are one contiguous span: 16-byte chunks.
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int row0 = qc + wq0;
          uint16_t* dst = obase + (int64_t)row0 * D;
          constexpr int NCO = NQB * 16 * D / 8;
          for (int c = lane; c < NCO; c += 64)
            if (row0 + c * 8 / D < a.Nq)
              __builtin_nontemporal_store(*(const u32x4*)(stage + c * 8), (u32x4*)(dst + c * 8));
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
      if (!more) break;
      qc = qn;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  } else {
    if (q0 + wq0 < a.Nq) {
      qk(Ks, s_cur);
      tile(0, std::false_type{});
      qk(Ks + C::K_ELEMS, s_cur, RFAST ? 4 : min(4, (a.Nk - BN + 15) / 16));
      tile(1, std::true_type{});
    }
  }
  } else {
  store_k(0, 0);
  store_v(0);
  __syncthreads();
  // Tile t+1 streams from HBM into registers while tile t is computed, and
  // is stored into the other LDS stage afterwards.  The last tile is peeled
  // (it alone may hold keys past Nk).
  // A wave whose queries all lie past Nq only helps with the tile loads.
  const bool active = q0 + wq0 < a.Nq;
  for (int t = 0; t + 1 < ntiles; ++t) {
    load_k(t + 1);
    load_v(t + 1);
    if (active) {
      qk(Ks + (t & 1) * C::K_ELEMS, s_cur);
      tile(t, std::false_type{});
    }
    store_k((t + 1) & 1, t + 1);
    store_v((t + 1) & 1);
    __syncthreads();
  }
  if (active) {
    const int klast = (ntiles - 1) * BN;
    qk(Ks + ((ntiles - 1) & 1) * C::K_ELEMS, s_cur, RFAST ? 4 : min(4, (a.Nk - klast + 15) / 16));
    tile(ntiles - 1, std::true_type{});
  }
  }

  // Epilogue: normalise by the row sum (row D of O^T, held by lane group
  // (D%16)/4) and store O (lane holds O[q][cb*16 + g*4 .. +3]).
  uint16_t* obase = (uint16_t*)a.o + tok_base(a, a.o_sb, a.o_sh, b, h);
  // Row log-sum-exp (natural log) of query qi: m is the row's reference in
  // log2 units, lsum the row sum against it; one lane group writes it.
  auto write_lse = [&](int qb, float lsum, int qi) {
    if (a.lse && g == 0 && qi < a.Nq) {
      const uint32_t row = tok_row(a, 1, b, qi);
      if (row != kPadTok) {
        const int64_t ntok = a.image ? (int64_t)a.img_h * a.img_w : a.Nq;
        const int img = a.image ? fdiv(b, a.fd_nw) : b;
        a.lse[((int64_t)img * a.H + h) * ntok + row] = (m[qb] + __builtin_amdgcn_logf(lsum)) * kLn2;
      }
    }
  };
  constexpr int LB = D / 16, LG = (D % 16) / 4, LR = D % 4;
#ifndef ATTN_STAGE_O
#define ATTN_STAGE_O 1
#endif
  // Two-tile form over one query tile (batched layout at d = 64) with rows
  // stored back to back: a wave's NQB*16 output rows are one contiguous
  // span.  It is staged through LDS (the K/V stages are free by now) and
  // stored as 16-byte chunks, so each streaming store covers whole lines
  // instead of 8-byte pieces of four rows.
  if constexpr (ATTN_STAGE_O && TWO && !IMG && !kPersist && D % 8 == 0) {
    if (a.o_sn == D && ((a.o_sb | a.o_sh) & 7) == 0) {
      static_assert((size_t)NW * NQB * 16 * D * 2 <= C::KV_BYTES, "O staging must fit the K/V stages");
      __syncthreads();  // every wave has finished reading K and V
      uint16_t* stage = (uint16_t*)lds + wave * (NQB * 16 * D);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float lsum;
        if constexpr (C::ONES) lsum = __shfl(o[LB < CB ? LB : 0][qb][LR], LG * 16 + l16);
        else lsum = sum_across_groups(l[qb]);
        const float inv = (F8 ? a.v_descale : 1.f) / lsum;
        const int r = qb * 16 + (kLean ? lane_id_here() & 15 : l16);
        write_lse(qb, lsum, q0 + wq0 + r);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int c0 = cb * 16 + g * 4;
          if (c0 < D) {
            const f32x4 v = o[cb][qb] * inv;
            *(u32x2*)(stage + r * D + c0) = u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int row0 = q0 + wq0;
      uint16_t* dst = obase + (int64_t)row0 * D;
      constexpr int NCH = NQB * 16 * D / 8;  // 16-byte chunks of the span
      for (int c = lane_id_here(); c < NCH; c += 64) {
        if (row0 + c * 8 / D < a.Nq)  // rows past Nq are not stored
          __builtin_nontemporal_store(*(const u32x4*)(stage + c * 8), (u32x4*)(dst + c * 8));
      }
      return;
    }
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float lsum;
    if constexpr (C::ONES) lsum = __shfl(o[LB < CB ? LB : 0][qb][LR], LG * 16 + l16);
    else lsum = sum_across_groups(l[qb]);
    const float inv = (F8 ? a.v_descale : 1.f) / lsum;
    const int qi = q0 + wq0 + qb * 16 + (kLean ? lane_id_here() & 15 : l16);
    write_lse(qb, lsum, qi);
    const uint32_t off = qi < a.Nq ? tok_row(a, a.o_sn, b, qi) : kPadTok;
    if (off != kPadTok) {  // rows past Nq and padding tokens are not stored
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c0 = cb * 16 + g * 4;
        if (c0 < D) {
          const f32x4 v = o[cb][qb] * inv;
          const u32x2 packed = {E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
          // Streaming (non-temporal) stores where O is most of the traffic
          // (cross-attention to a short context): measured faster there,
          // slower in the contraction form, neutral in the long-key forms.
          if constexpr (TWO) __builtin_nontemporal_store(packed, (u32x2*)(obase + off + c0));
          else *(u32x2*)(obase + off + c0) = packed;
        }
      }
    }
  }
}

}  // namespace attn

#endif  // ATTN_MFMA_H_
