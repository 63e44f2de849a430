// One compiled instance of the attention kernels, selected by INST_DT (an
// attn_dtype_t value) and INST_D (head dim, or the fp32 register bucket).
#include "attn_device.h"
#include "attn_mfma.h"
#include "attn_win.h"
#include "attn_launch.h"

#ifndef INST_DT
#error "INST_DT must be defined"
#endif
#ifndef INST_D
#error "INST_D must be defined"
#endif

namespace attn {
namespace {

constexpr size_t kMaxLds = 160 * 1024;

template <typename K>
int launch_kernel(K kernel, int threads, int bm, size_t dyn, AttnArgs a, hipStream_t s) {
  a.n_qtiles = (a.Nq + bm - 1) / bm;
  a.fd_qt = make_fastdiv(a.n_qtiles);
  const int64_t blocks = (int64_t)a.n_qtiles * a.H * a.B;
  if (blocks > 0x7fffffff) return ATTN_E_UNSUPPORTED;
  if (dyn > kMaxLds) return ATTN_E_UNSUPPORTED;
  a.n_blocks = (int)blocks;
  if (dyn > 32 * 1024 &&
      hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn) !=
          hipSuccess)
    return ATTN_E_LAUNCH;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(threads), dyn, s, a);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

#if INST_DT == 0
template <int BIAS, bool MASK>
int launch_one(const AttnArgs& a, hipStream_t s) {
  // Windows of at most 64 tokens: one workgroup per (window, head) unit on
  // the fp32 matrix instructions.
  if constexpr (BIAS != ATTN_BIAS_RELPOS) {
    if (a.Nq <= 64 && a.Nk <= 64) {
      AttnArgs w = a;
      w.n_qtiles = 1;
      w.fd_qt = make_fastdiv(1);
      const int64_t blocks = (int64_t)a.B * a.H;
      if (blocks > 0x7fffffff) return ATTN_E_UNSUPPORTED;
      w.n_blocks = (int)blocks;
      const size_t dyn = win_lds_bytes(a, WinCfgF32<INST_D>::KV_BYTES);
      if (dyn > kMaxLds) return ATTN_E_UNSUPPORTED;
      auto kern = !MASK ? attn_fwd_win<F32E, INST_D, BIAS, ATTN_MASK_NONE>
                  : a.mask_kind == ATTN_MASK_ADDITIVE ? attn_fwd_win<F32E, INST_D, BIAS, ATTN_MASK_ADDITIVE>
                                                      : attn_fwd_win<F32E, INST_D, BIAS, ATTN_MASK_SHIFT_REGIONS>;
      if (dyn > 32 * 1024 &&
          hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn) !=
              hipSuccess)
        return ATTN_E_LAUNCH;
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kWinWaves * 64), dyn, s, w);
      return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
    }
  }
  constexpr size_t st = 2 * (size_t)kF32BN * INST_D * 4;
  if (dyn_lds_bytes(a, kF32Threads) + st > kMaxLds) return ATTN_E_UNSUPPORTED;
  return launch_kernel(attn_fwd_f32<INST_D, BIAS, MASK>, kF32Threads, kF32Threads,
                       dyn_lds_bytes(a, kF32Threads), a, s);
}
#else
#if INST_DT == 2
using Elem = BF16;
#else
using Elem = F16;
#endif
constexpr int kNW = 4;
#ifndef ATTN_NQB
#define ATTN_NQB 2  // 16-query blocks per wave
#endif
constexpr int kNQB = ATTN_NQB;

// The tiled kernel in the instance for the call's layout (the ping-pong
// form, NW = 8 with a relative-position row form, exists for the batched
// layout only).
template <int BIAS, bool MASK, int RMODE, int WPE, int NW = kNW>
int launch_mfma(const AttnArgs& a, hipStream_t s) {
  constexpr int D = INST_D;
  using C = MfmaCfg<D, NW, kNQB>;
  const size_t lds = mfma_lds_bytes<D, NW, kNQB, RMODE>(a);
  constexpr bool kPingPong = NW == 8 && RMODE != kTwoTiles;
  if constexpr (!kPingPong) {
    if (a.image)
      return launch_kernel(attn_fwd_mfma<Elem, D, NW, kNQB, BIAS, MASK, RMODE, WPE, true>, C::NT, C::BM, lds, a, s);
  }
  return launch_kernel(attn_fwd_mfma<Elem, D, NW, kNQB, BIAS, MASK, RMODE, WPE, false>, C::NT, C::BM, lds, a, s);
}

template <int BIAS, bool MASK>
int launch_one(const AttnArgs& a, hipStream_t s) {
  constexpr int D = INST_D;
  using C = MfmaCfg<D, kNW, kNQB>;
  // Windows of at most 64 tokens: one wave per (window, head) unit.
  if constexpr (BIAS != ATTN_BIAS_RELPOS) {
    if (a.Nq <= 64 && a.Nk <= 64) {
      AttnArgs w = a;
      w.n_qtiles = 1;
      w.fd_qt = make_fastdiv(1);
      const int64_t blocks = (int64_t)a.B * a.H;
      if (blocks > 0x7fffffff) return ATTN_E_UNSUPPORTED;
      w.n_blocks = (int)blocks;
      const size_t dyn = win_lds_bytes(a, WinCfg<D>::KV_BYTES);
      if (dyn > kMaxLds) return ATTN_E_UNSUPPORTED;
      auto kern = !MASK ? attn_fwd_win<Elem, D, BIAS, ATTN_MASK_NONE>
                  : a.mask_kind == ATTN_MASK_ADDITIVE ? attn_fwd_win<Elem, D, BIAS, ATTN_MASK_ADDITIVE>
                                                      : attn_fwd_win<Elem, D, BIAS, ATTN_MASK_SHIFT_REGIONS>;
      if (dyn > 32 * 1024 &&
          hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn) !=
              hipSuccess)
        return ATTN_E_LAUNCH;
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kWinWaves * 64), dyn, s, w);
      return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
    }
  }
  // Waves per SIMD the register allocation targets: the most that still
  // fit the tile state without spilling (checked per head dim).
#ifdef ATTN_WPE  // one occupancy target for every path (tuning builds)
  constexpr int kWpeNone = ATTN_WPE, kWpeRelpos = ATTN_WPE, kWpeAug = ATTN_WPE;
#else
  constexpr int kWpeNone = D <= 32 ? 4 : (D <= 40 ? 3 : 2);
  constexpr int kWpeRelpos = D <= 40 ? 3 : 2;
#ifdef ATTN_WPE_AUG
  constexpr int kWpeAug = ATTN_WPE_AUG;
#else
  constexpr int kWpeAug = D <= 64 ? 3 : 2;
#endif
#endif
#ifndef ATTN_PP
#define ATTN_PP 1
#endif
#ifndef ATTN_PP_MIN_KEYS
#define ATTN_PP_MIN_KEYS 1024
#endif
  // Long key ranges with the 64-wide relative-position row form: eight-wave
  // workgroups whose two wave groups alternate matrix and softmax phases
  // (measured faster there; without a bias the four-wave kernel is faster).
  // The row and contraction forms take equal query and key grids; keys on a
  // grid of their own go to the general table form.
  [[maybe_unused]] const bool rel_same_grid = a.gh == a.kgh && a.gw == a.kgw;
  if constexpr (ATTN_PP && !MASK && BIAS == ATTN_BIAS_RELPOS) {
    if (rel_same_grid && a.gw == 64 && a.Nk >= ATTN_PP_MIN_KEYS && a.Nq >= 256 && !a.image) {
      return launch_mfma<BIAS, false, kRelRow64, 2, 8>(a, s);
    }
  }
  // Relative position: 64-wide grids take the row form, grids with
  // gh + gw <= 32 fold the bias into the QK^T contraction.
  if constexpr (BIAS == ATTN_BIAS_RELPOS && !MASK) {
    if (rel_same_grid && a.gw == 64) return launch_mfma<BIAS, false, kRelRow64, kWpeRelpos>(a, s);
    if (rel_same_grid && a.gh + a.gw <= 32) return launch_mfma<BIAS, false, kRelAug, kWpeAug>(a, s);
  }
  constexpr int wpe = (BIAS == ATTN_BIAS_NONE && !MASK) ? kWpeNone : 1;
  // Keys spanning exactly two tiles (cross-attention to short contexts):
  // both tiles are loaded with the queries, one barrier, no waits between.
#ifndef ATTN_WPE_TWO
#define ATTN_WPE_TWO (D <= 40 ? 4 : (D <= 64 ? 3 : 2))
#endif
  if constexpr (BIAS == ATTN_BIAS_NONE && !MASK) {
    constexpr int kWpeTwo = ATTN_WPE_TWO;
    // Eight-wave workgroups (256 queries share one K/V load) where the wave
    // target is even, so that whole workgroups fill each CU.
    constexpr int kTwoNW = kWpeTwo % 2 == 0 ? 8 : 4;
    if (a.Nk > C::BN && a.Nk <= 2 * C::BN) return launch_mfma<BIAS, MASK, kTwoTiles, kWpeTwo, kTwoNW>(a, s);
  }
  return launch_mfma<BIAS, MASK, kRelTables, wpe>(a, s);
}
#endif

}  // namespace

template <>
int launch_inst<INST_DT, INST_D>(const AttnArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const bool mask = a.mask_kind != ATTN_MASK_NONE;
  switch (a.bias_kind) {
    case ATTN_BIAS_NONE:
      return mask ? launch_one<ATTN_BIAS_NONE, true>(a, s) : launch_one<ATTN_BIAS_NONE, false>(a, s);
    case ATTN_BIAS_TABLE:
      return mask ? launch_one<ATTN_BIAS_TABLE, true>(a, s) : launch_one<ATTN_BIAS_TABLE, false>(a, s);
    case ATTN_BIAS_RELPOS:
      return mask ? launch_one<ATTN_BIAS_RELPOS, true>(a, s) : launch_one<ATTN_BIAS_RELPOS, false>(a, s);
    default:
      return mask ? launch_one<ATTN_BIAS_ADDITIVE, true>(a, s)
                  : launch_one<ATTN_BIAS_ADDITIVE, false>(a, s);
  }
}

}  // namespace attn
