// Fused scaled-dot-product attention forward for gfx950 (CDNA4).
//
//   O = softmax(scale * Q K^T + bias + mask) V
//
// The attention map is never written to memory: a workgroup owns a tile of
// queries of one (batch item, head), streams key/value tiles through LDS and
// keeps the running row maximum, row sum and output accumulator in registers
// (online softmax).  Operator fusion keeps intermediate results in registers
// and shared memory instead of global memory ("Training and inference
// acceleration for large vision models", section 2); the window
// partition/shift/reverse of Swin are index mappings (same section) and are
// folded into the load/store addresses here.
//
// Half-precision path: both contractions run on v_mfma_f32_16x16x32_{bf16,f16}.
// The score tile is computed transposed, S^T = K Q^T, so that in the MFMA
// accumulator layout each lane holds scores of ONE query (column lane%16) for
// 4 keys per 16x16 block: row statistics need only two cross-lane steps, the
// softmax rescale of the output accumulator is one scalar per lane, and the
// probabilities are already in the B-operand layout of O^T += V^T P^T (the
// key order inside a 32-key chunk is permuted, and V^T is stored in LDS with
// the same permutation).
#ifndef ATTN_DEVICE_H_
#define ATTN_DEVICE_H_
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/attn.h"
#include "attn_internal.h"
#include "attn_plan.h"

namespace attn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element types
// ---------------------------------------------------------------------------
struct BF16 {
  static __device__ __forceinline__ uint16_t one_bits() { return 0x3f80; }
  static __device__ __forceinline__ float to_f(uint16_t x) {
    return __uint_as_float((uint32_t)x << 16);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // c + a.lo*b.lo + a.hi*b.hi of two packed pairs, in fp32 (v_dot2_f32_bf16).
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
  }
};

struct F16 {
  static __device__ __forceinline__ uint16_t one_bits() { return 0x3c00; }
  static __device__ __forceinline__ float to_f(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // c + a.lo*b.lo + a.hi*b.hi of two packed pairs, in fp32 (v_dot2_f32_f16).
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  }
};

template <class E>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  return E::to_f(((const uint16_t*)p)[i]);
}
struct F32E {};
template <>
__device__ __forceinline__ float load_elem<F32E>(const void* p, int64_t i) {
  return ((const float*)p)[i];
}

// Eight E4M3 codes (one per byte, in order) -> the eight elements of E they
// encode.  Every E4M3 value is exact in f16 and in bf16, so the widening is
// exact; gfx950 converts the OCP E4M3 format (bias 7, S.1111.111 = NaN) with
// v_cvt_scalef32_pk_{f16,bf16}_fp8, two codes per instruction (scale 1).
template <class E>
__device__ __forceinline__ u32x4 widen_e4m3(u32x2 w) {
  if constexpr (std::is_same<E, F16>::value) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.f, true))};
  } else {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, true))};
  }
}

// Dot product of 4 consecutive elements of two arrays (8-byte / 16-byte loads).
template <class E>
__device__ __forceinline__ float dot4(const void* x, int64_t i, const void* y, int64_t j) {
  const u32x2 a = *(const u32x2*)((const uint16_t*)x + i);
  const u32x2 b = *(const u32x2*)((const uint16_t*)y + j);
  float r = E::to_f(a[0] & 0xffff) * E::to_f(b[0] & 0xffff);
  r = fmaf(E::to_f(a[0] >> 16), E::to_f(b[0] >> 16), r);
  r = fmaf(E::to_f(a[1] & 0xffff), E::to_f(b[1] & 0xffff), r);
  return fmaf(E::to_f(a[1] >> 16), E::to_f(b[1] >> 16), r);
}
template <>
__device__ __forceinline__ float dot4<F32E>(const void* x, int64_t i, const void* y, int64_t j) {
  const f32x4 a = *(const f32x4*)((const float*)x + i);
  const f32x4 b = *(const f32x4*)((const float*)y + j);
  return fmaf(a[3], b[3], fmaf(a[2], b[2], fmaf(a[1], b[1], a[0] * b[0])));
}

// n / d for 0 <= n < 2^31 with host-computed constants (multiply-high, add,
// shift; scalar instructions when n is uniform).
__device__ __forceinline__ int fdiv(int n, FastDiv f) {
  const uint32_t hi = (uint32_t)(((uint64_t)(uint32_t)n * f.mul) >> 32);
  return (int)((hi + (uint32_t)n) >> f.shift);
}

// ---------------------------------------------------------------------------
// Workgroup renumbering for the 8 XCDs of MI355X.  The dispatcher hands
// workgroup i to XCD i % 8, and each XCD has its own L2.  The logical id
// returned here gives every XCD one contiguous range of ids, so tiles that
// read the same data (the query tiles of one (batch item, head), which all
// stream the same K/V; neighbouring windows, which share cache lines of an
// image row) are processed by one XCD at about the same time and fetch the
// shared lines from HBM once.  A bijection on [0, n) for any n.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_logical_id(int i, int n) {
  constexpr int kXcds = 8;
  const int per = n / kXcds, extra = n % kXcds;
  const int x = i % kXcds, local = i / kXcds;
  return x * per + (x < extra ? x : extra) + local;
}

// ---------------------------------------------------------------------------
// Token addressing: batched layout, or image layout with zero padding, the
// window partition and the cyclic shift folded in.  The image is padded at
// the bottom and right to pimg_h x pimg_w (whole windows); window w of image
// img, token t of the window reads shifted padded pixel (wy*win_h+ty,
// wx*win_w+tx), which holds padded pixel ((y+shift_h) mod pimg_h,
// (x+shift_w) mod pimg_w); a padded pixel past the image is a padding token
// (zero q, k, v; its output is not stored).  Stores use the same map, which
// is the reverse partition, reverse shift and crop.
// ---------------------------------------------------------------------------
// Image pixel index of window token (ty, tx) whose window starts at shifted
// padded pixel (y0, x0), or -1 for a padding token.
__device__ __forceinline__ int image_pixel(const AttnArgs& a, int y0, int x0, int ty, int tx) {
  int y = y0 + ty + a.shift_h;
  if (y >= a.pimg_h) y -= a.pimg_h;
  int x = x0 + tx + a.shift_w;
  if (x >= a.pimg_w) x -= a.pimg_w;
  return (y < a.img_h && x < a.img_w) ? y * a.img_w + x : -1;
}

// Full element offset of token t of batch item b, head h; -1 for a padding
// token.
__device__ __forceinline__ int64_t tok_off(const AttnArgs& a, int64_t sb, int64_t sh, int64_t sn,
                                           int b, int h, int t) {
  if (!a.image) return (int64_t)b * sb + (int64_t)h * sh + (int64_t)t * sn;
  const int img = fdiv(b, a.fd_nw);
  const int w = b - img * a.nw;
  const int wy = fdiv(w, a.fd_nwx), wx = w - wy * a.nwx;
  const int ty = fdiv(t, a.fd_win_w), tx = t - ty * a.win_w;
  const int pix = image_pixel(a, wy * a.win_h, wx * a.win_w, ty, tx);
  return pix < 0 ? -1 : (int64_t)img * sb + (int64_t)h * sh + (int64_t)pix * sn;
}

// The same map split into a per-(batch item, head) base (uniform across a
// workgroup) and a 32-bit per-token offset (kPadTok for a padding token);
// the host guarantees every in-slice offset fits in 31 bits (29 in the
// image layout).
__device__ __forceinline__ int64_t tok_base(const AttnArgs& a, int64_t sb, int64_t sh, int b, int h) {
  const int img = a.image ? fdiv(b, a.fd_nw) : b;
  return (int64_t)img * sb + (int64_t)h * sh;
}
__device__ __forceinline__ uint32_t tok_row(const AttnArgs& a, int64_t sn, int b, int t) {
  if (!a.image) return (uint32_t)t * (uint32_t)sn;
  const int w = b - fdiv(b, a.fd_nw) * a.nw;
  const int wy = fdiv(w, a.fd_nwx), wx = w - wy * a.nwx;
  const int ty = fdiv(t, a.fd_win_w), tx = t - ty * a.win_w;
  const int pix = image_pixel(a, wy * a.win_h, wx * a.win_w, ty, tx);
  return pix < 0 ? kPadTok : (uint32_t)pix * (uint32_t)sn;
}

// Region (0..8) of token t of window w in the shifted padded image
// (SHIFT_REGIONS).
__device__ __forceinline__ int region_of(const AttnArgs& a, int w, int t) {
  const int wy = fdiv(w, a.fd_nwx), wx = w - wy * a.nwx;
  const int ty = fdiv(t, a.fd_win_w), tx = t - ty * a.win_w;
  const int y = wy * a.win_h + ty, x = wx * a.win_w + tx;
  const int ry = y < a.pimg_h - a.win_h ? 0 : (y < a.pimg_h - a.shift_h ? 1 : 2);
  const int rx = x < a.pimg_w - a.win_w ? 0 : (x < a.pimg_w - a.shift_w ? 1 : 2);
  return 3 * ry + rx;
}


// Relative-position table row of query coordinate qc and key coordinate kc
// on an axis of qn query and kn key positions: the shorter axis is
// stretched onto the longer one and the scaled difference floored, so that
// rows run from 0 to at most 2*max(qn, kn)-2 (equal axes: qc - kc + kn - 1).
__device__ __forceinline__ int rel_row(int qc, int kc, int qn, int kn) {
  if (qn == kn) return qc - kc + kn - 1;
  if (qn > kn) return qc + (kn - 1 - kc) * qn / kn;
  return qc * kn / qn + (kn - 1 - kc);
}

// Row r of a relative-position table resized from n stored to m needed rows
// (linear interpolation along the offset axis, end rows kept): the value is
// (1-f)*T[i0] + f*T[i1] at position r*(n-1)/(m-1), with i0 = floor and the
// fraction from exact integer arithmetic.  n == m gives row r itself.
__device__ __forceinline__ void resized_row(int r, int n, int m, int& i0, int& i1, float& f) {
  if (n == m || n == 1 || m == 1) {
    i0 = i1 = n == m ? r : 0;
    f = 0.f;
    return;
  }
  const int num = r * (n - 1);
  i0 = num / (m - 1);
  i1 = i0 + 1 < n ? i0 + 1 : i0;
  f = (float)(num - i0 * (m - 1)) * __builtin_amdgcn_rcpf((float)(m - 1));
}

// ---------------------------------------------------------------------------
// Bias and mask, evaluated per (query, key) from on-chip index data.
//
// LDS layout (dynamic):  kinfo[Nk] (when any index-based term is present),
// then either the head's table column [(2gh-1)(2gw-1)] or relh[gh][BM],
// relw[gw][BM] (relative-position terms of this workgroup's queries).  All
// stored values are pre-multiplied by log2(e): the softmax runs in base 2.
// kinfo[j] = kh | kw << 11 | region << 22.
// ---------------------------------------------------------------------------
struct BiasCtx {
  const int* kinfo;
  const float* tbl;   // TABLE
  const float* relh;  // RELPOS [kgh][BM]
  const float* relw;  // RELPOS [kgw][BM]
};

// Fill kinfo and the table / relative-position terms.  `E` is the element
// type of the tables and of q (relative-position terms use the raw query).
// RELPOS_VALU: compute the relative-position tables here with plain dot
// products (the fp32 kernel); the MFMA kernel fills them itself.
template <class E, int BIAS, bool MASK, int BM, int NT, bool RELPOS_VALU = true>
__device__ void setup_bias(const AttnArgs& a, char* dyn, int b, int h, int q0, BiasCtx& bc) {
  const int tid = __builtin_amdgcn_workitem_id_x();
  char* p = dyn;
  bc.kinfo = nullptr;
  bc.tbl = bc.relh = bc.relw = nullptr;
  if (needs_kinfo(BIAS, MASK)) {
    int* kinfo = (int*)p;
    const int w = a.nw ? b - fdiv(b, a.fd_nw) * a.nw : 0;
    for (int j = tid; j < a.Nk; j += NT) {
      int v = 0;
      if (BIAS == ATTN_BIAS_TABLE || BIAS == ATTN_BIAS_RELPOS) {
        const int kh = fdiv(j, a.fd_kgw);
        v = kh | ((j - kh * a.kgw) << 11);
      }
      if (MASK && a.mask_kind == ATTN_MASK_SHIFT_REGIONS) v |= region_of(a, w, j) << 22;
      kinfo[j] = v;
    }
    bc.kinfo = kinfo;
    p += ((size_t)a.Nk * 4 + 15) / 16 * 16;
  }
  if (BIAS == ATTN_BIAS_TABLE) {
    float* tbl = (float*)p;
    const int n = (2 * a.gh - 1) * (2 * a.gw - 1);
    for (int r = tid; r < n; r += NT) tbl[r] = load_elem<E>(a.table, (int64_t)r * a.H + h) * kLog2e;
    bc.tbl = tbl;
  }
  if (BIAS == ATTN_BIAS_RELPOS) {
    // relh[kh][i] = q_i . Rh[rel_row(qh_i, kh)], relw[kw][i] = q_i . Rw[rel_row(qw_i, kw)]
    // for the kgh x kgw key grid (equal grids: Rh[qh_i - kh + gh - 1]).
    float* relh = (float*)p;
    float* relw = relh + a.kgh * BM;
    const int nk = a.kgh + a.kgw;
    for (int e = tid; RELPOS_VALU && e < BM * nk; e += NT) {
      const int il = e % BM, kk = e / BM;
      const int qi = min(q0 + il, a.Nq - 1);
      const int qh = fdiv(qi, a.fd_gw), qw = qi - qh * a.gw;
      const int64_t qo = tok_off(a, a.q_sb, a.q_sh, a.q_sn, b, h, qi);
      const bool hax = kk < a.kgh;
      const int r = hax ? rel_row(qh, kk, a.gh, a.kgh) : rel_row(qw, kk - a.kgh, a.gw, a.kgw);
      const int need = hax ? 2 * max(a.gh, a.kgh) - 1 : 2 * max(a.gw, a.kgw) - 1;
      int i0, i1;
      float f;
      resized_row(r, hax ? a.rh_rows : a.rw_rows, need, i0, i1, f);
      const void* tb = hax ? a.rh : a.rw;
      float acc0 = 0.f, acc1 = 0.f;  // a padding query (qo < 0) is zero
      for (int c = 0; qo >= 0 && c < a.D; c += 4) {
        acc0 += dot4<E>(a.q, qo + c, tb, (int64_t)i0 * a.D + c);
        if (i1 != i0) acc1 += dot4<E>(a.q, qo + c, tb, (int64_t)i1 * a.D + c);
      }
      const float acc = i1 != i0 ? acc0 + f * (acc1 - acc0) : acc0;
      (hax ? relh + kk * BM : relw + (kk - a.kgh) * BM)[il] = acc * kLog2e;
    }
    bc.relh = relh;
    bc.relw = relw;
  }
}

// Per-query constants for the bias of one query row.
struct QInfo {
  int il;      // row inside the workgroup's query tile
  int qi;      // query index, clamped to Nq-1
  int tab;     // TABLE: (qh+gh-1)*(2gw-1) + qw+gw-1
  int region;  // SHIFT_REGIONS
};

template <int BIAS, bool MASK>
__device__ __forceinline__ QInfo make_qinfo(const AttnArgs& a, int b, int qi, int il) {
  QInfo qinf;
  qinf.il = il;
  qinf.qi = qi;
  qinf.tab = 0;
  qinf.region = 0;
  if (BIAS == ATTN_BIAS_TABLE) {
    const int qh = fdiv(qi, a.fd_gw), qw = qi - qh * a.gw;
    qinf.tab = (qh + a.gh - 1) * (2 * a.gw - 1) + qw + a.gw - 1;
  }
  if (MASK && a.mask_kind == ATTN_MASK_SHIFT_REGIONS) qinf.region = region_of(a, b - fdiv(b, a.fd_nw) * a.nw, qi);
  return qinf;
}

// (bias + mask) * log2(e) for query `qinf` and key kj (kj < Nk).
template <class E, int BIAS, bool MASK, int BM>
__device__ __forceinline__ float bias_log2(const AttnArgs& a, const BiasCtx& bc, const QInfo& qinf,
                                           int b, int kj) {
  float r = 0.f;
  int ki = 0;
  if (needs_kinfo(BIAS, MASK)) ki = bc.kinfo[kj];
  if (BIAS == ATTN_BIAS_TABLE) {
    const int kh = ki & 2047, kw = (ki >> 11) & 2047;
    r += bc.tbl[qinf.tab - (kh * (2 * a.gw - 1) + kw)];
  } else if (BIAS == ATTN_BIAS_RELPOS) {
    const int kh = ki & 2047, kw = (ki >> 11) & 2047;
    r += bc.relh[kh * BM + qinf.il] + bc.relw[kw * BM + qinf.il];
  } else if (BIAS == ATTN_BIAS_ADDITIVE) {
    const int64_t off = (int64_t)(b % a.badd_n) * a.badd_s0 + (int64_t)qinf.qi * a.badd_s1 + kj;
    r += load_elem<E>(a.badd, off) * kLog2e;
  }
  if (MASK) {
    if (a.mask_kind == ATTN_MASK_SHIFT_REGIONS) {
      if ((ki >> 22) != qinf.region) r += a.mask_value * kLog2e;
    } else {
      const int64_t off = (int64_t)(b % a.madd_n) * a.madd_s0 + (int64_t)qinf.qi * a.madd_s1 + kj;
      r += load_elem<E>(a.madd, off) * kLog2e;
    }
  }
  return r;
}

// ---------------------------------------------------------------------------
// fp32 kernel: one thread per query, key/value tiles broadcast from LDS.
// ---------------------------------------------------------------------------
template <int DMAX, int BIAS, bool MASK>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32(AttnArgs a) {
  constexpr int BM = kF32Threads;
  __shared__ __attribute__((aligned(16))) float Ks[kF32BN][DMAX];
  __shared__ __attribute__((aligned(16))) float Vs[kF32BN][DMAX];
  extern __shared__ __attribute__((aligned(16))) char dyn_lds[];

  const int tid = __builtin_amdgcn_workitem_id_x();
  int bid = xcd_logical_id(__builtin_amdgcn_workgroup_id_x(), a.n_blocks);
  const int qt_div = fdiv(bid, a.fd_qt);
  const int qt = bid - qt_div * a.n_qtiles;
  const int b = fdiv(qt_div, a.fd_h);
  const int h = qt_div - b * a.H;
  const int q0 = qt * BM;
  const int D = a.D;

  BiasCtx bc;
  setup_bias<F32E, BIAS, MASK, BM, kF32Threads>(a, dyn_lds, b, h, q0, bc);

  const int qi = min(q0 + tid, a.Nq - 1);
  const QInfo qinf = make_qinfo<BIAS, MASK>(a, b, qi, tid);
  float qv[DMAX], acc[DMAX];
  {
    const int64_t qo = tok_off(a, a.q_sb, a.q_sh, a.q_sn, b, h, qi);
    const float* qp = (const float*)a.q + (qo < 0 ? 0 : qo);
#pragma unroll
    for (int c = 0; c < DMAX; c += 4) {
      const f32x4 v = c < D && qo >= 0 ? *(const f32x4*)(qp + c) : f32x4{0.f, 0.f, 0.f, 0.f};
      qv[c] = v[0]; qv[c + 1] = v[1]; qv[c + 2] = v[2]; qv[c + 3] = v[3];
      acc[c] = acc[c + 1] = acc[c + 2] = acc[c + 3] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * kLog2e;
  const int ntiles = (a.Nk + kF32BN - 1) / kF32BN;
  const int rch = D / 4;
  // Columns D..DMAX of the tiles are never loaded: zero them once, so the
  // dot products below run over DMAX columns without per-column branches.
  for (int i = tid; i < kF32BN * (DMAX - D); i += kF32Threads) {
    const int row = i / (DMAX - D), col = D + i % (DMAX - D);
    Ks[row][col] = 0.f;
    Vs[row][col] = 0.f;
  }
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    for (int ch = tid; ch < kF32BN * rch; ch += kF32Threads) {
      const int row = ch / rch, col = (ch % rch) * 4;
      const int key = t * kF32BN + row;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < a.Nk) {
        const int64_t ko = tok_off(a, a.k_sb, a.k_sh, a.k_sn, b, h, key);
        const int64_t vo = tok_off(a, a.v_sb, a.v_sh, a.v_sn, b, h, key);
        if (ko >= 0) kv = *(const f32x4*)((const float*)a.k + ko + col);  // padding keys stay zero
        if (vo >= 0) vv = *(const f32x4*)((const float*)a.v + vo + col);
      }
      *(f32x4*)&Ks[row][col] = kv;
      *(f32x4*)&Vs[row][col] = vv;
    }
    __syncthreads();
    float s[kF32BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      const int kj = t * kF32BN + j;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < DMAX; c += 4) {
        const f32x4 kv = *(const f32x4*)&Ks[j][c];
        dot = fmaf(qv[c], kv[0], dot);
        dot = fmaf(qv[c + 1], kv[1], dot);
        dot = fmaf(qv[c + 2], kv[2], dot);
        dot = fmaf(qv[c + 3], kv[3], dot);
      }
      float v = dot * sl2;
      if (BIAS != ATTN_BIAS_NONE || MASK)
        v += bias_log2<F32E, BIAS, MASK, BM>(a, bc, qinf, b, min(kj, a.Nk - 1));
      if (kj >= a.Nk) v = -INFINITY;
      s[j] = v;
      mx = fmaxf(mx, v);
    }
    const float mnew = fmaxf(m, mx);
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < DMAX; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      const float p = __builtin_amdgcn_exp2f(s[j] - mref);
      l += p;
#pragma unroll
      for (int c = 0; c < DMAX; c += 4) {
        const f32x4 vv = *(const f32x4*)&Vs[j][c];
        acc[c] = fmaf(p, vv[0], acc[c]);
        acc[c + 1] = fmaf(p, vv[1], acc[c + 1]);
        acc[c + 2] = fmaf(p, vv[2], acc[c + 2]);
        acc[c + 3] = fmaf(p, vv[3], acc[c + 3]);
      }
    }
  }
  const int64_t oo = q0 + tid < a.Nq ? tok_off(a, a.o_sb, a.o_sh, a.o_sn, b, h, q0 + tid) : -1;
  if (oo >= 0) {  // rows past Nq and padding tokens are not stored
    const float inv = 1.f / l;
    float* op = (float*)a.o + oo;
#pragma unroll
    for (int c = 0; c < DMAX; c += 4)
      if (c < D) *(f32x4*)(op + c) = f32x4{acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
  }
}

}  // namespace attn

#endif  // ATTN_DEVICE_H_
