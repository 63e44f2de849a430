// One compiled instance of the attention kernels, selected by INST_DT (an
// attn_dtype_t value) and INST_D (head dim, or the fp32 register bucket).
// The kernel and its form come from the call's plan (attn_plan.h), the same
// computation the host validation ran.
#include "attn_device.h"
#include "attn_mfma.h"
#include "attn_win.h"
#include "attn_bwd.h"
#include "attn_launch.h"

#ifndef INST_DT
#error "INST_DT must be defined"
#endif
#ifndef INST_D
#error "INST_D must be defined"
#endif

namespace attn {
namespace {

template <typename K>
int launch_grid(K kernel, int threads, const Plan& p, const AttnArgs& a, hipStream_t s) {
  if (p.lds > 32 * 1024 &&
      hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds) !=
          hipSuccess)
    return ATTN_E_LAUNCH;
  hipLaunchKernelGGL(kernel, dim3((unsigned)p.blocks), dim3(threads), p.lds, s, a);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

// One workgroup per (window, head) unit.
template <class E, int DK, int BIAS, bool MASK, bool F8 = false>
int launch_win(const Plan& p, AttnArgs a, hipStream_t s) {
  a.n_qtiles = 1;
  a.fd_qt = make_fastdiv(1);
  a.n_blocks = (int)p.blocks;
  auto kern = !MASK ? attn_fwd_win<E, DK, BIAS, ATTN_MASK_NONE, F8>
              : a.mask_kind == ATTN_MASK_ADDITIVE ? attn_fwd_win<E, DK, BIAS, ATTN_MASK_ADDITIVE, F8>
                                                  : attn_fwd_win<E, DK, BIAS, ATTN_MASK_SHIFT_REGIONS, F8>;
  return launch_grid(kern, kWinWaves * 64, p, a, s);
}

#if INST_DT == 0
template <int BIAS, bool MASK>
int launch_one(const AttnArgs& a, hipStream_t s) {
  const Plan p = plan_f32<INST_D>(a);
  if (p.kernel < 0 || p.lds > kMaxLds || p.blocks > 0x7fffffff) return ATTN_E_UNSUPPORTED;
  if constexpr (BIAS != ATTN_BIAS_RELPOS) {
    // Windows of at most 64 tokens: one workgroup per (window, head) unit on
    // the fp32 matrix instructions.
    if (p.kernel == kKernWin) return launch_win<F32E, INST_D, BIAS, MASK>(p, a, s);
  }
  AttnArgs t = a;
  t.n_qtiles = (a.Nq + p.bm - 1) / p.bm;
  t.fd_qt = make_fastdiv(t.n_qtiles);
  t.n_blocks = (int)p.blocks;
  Plan dyn = p;
  dyn.lds = dyn_lds_bytes(a, kF32Threads);  // the K/V tiles are static LDS
  return launch_grid(attn_fwd_f32<INST_D, BIAS, MASK>, kF32Threads, dyn, t, s);
}
#else
#if INST_DT == 2
using Elem = BF16;
#else
using Elem = F16;
#endif

// The tiled kernel in the form and instance the plan names (the ping-pong
// form, NW = 8 with the row form, exists for the batched layout only).
template <int BIAS, bool MASK, int RMODE, int WPE, int NW = 4, bool F8 = false>
int launch_mfma(const Plan& p, const AttnArgs& a, hipStream_t s) {
  constexpr int D = INST_D;
  using C = MfmaCfg<D, NW, kNQB>;
  AttnArgs t = a;
  t.n_qtiles = (a.Nq + C::BM - 1) / C::BM;
  t.tpw = 1;
  if (RMODE == kTwoTiles && !a.image && two_tile_persists<D>()) {  // workgroups per unit, each over tpw query tiles
    t.tpw = p.tpw;
    t.n_qtiles = (t.n_qtiles + p.tpw - 1) / p.tpw;
  }
  t.fd_qt = make_fastdiv(t.n_qtiles);
  t.n_blocks = (int)p.blocks;
  constexpr bool kPingPong = NW == 8 && RMODE != kTwoTiles;
  if constexpr (!kPingPong) {
    if (a.image)
      return launch_grid(attn_fwd_mfma<Elem, D, NW, kNQB, BIAS, MASK, RMODE, WPE, true, F8>, C::NT, p, t, s);
  }
  return launch_grid(attn_fwd_mfma<Elem, D, NW, kNQB, BIAS, MASK, RMODE, WPE, false, F8>, C::NT, p, t, s);
}

// Waves per SIMD the register allocation of the tiled kernel targets: the
// most that still fit the tile state without spilling (checked per head dim).
constexpr int kWpeNone = INST_D <= 32 ? 4 : (INST_D <= 40 ? 3 : 2);
constexpr int kWpeRelpos = INST_D <= 40 ? 3 : 2;
constexpr int kWpeAug = INST_D <= 64 ? 3 : 2;

// 8-bit (E4M3) q, k, v: the window form or the tiled forms without relative
// position, with the loads widening the codes.
template <int BIAS, bool MASK>
int launch_f8(const Plan& p, const AttnArgs& a, hipStream_t s) {
  constexpr int D = INST_D;
  if (p.kernel == kKernWin) return launch_win<Elem, D, BIAS, MASK, true>(p, a, s);
  if (p.kernel != kKernMfma) return ATTN_E_UNSUPPORTED;
  if constexpr (BIAS == ATTN_BIAS_NONE && !MASK) {
    if (p.rmode == kTwoTiles)
      return launch_mfma<BIAS, MASK, kTwoTiles, two_tile_wpe<D>(), two_tile_nw<D>(), true>(p, a, s);
  }
  if (p.rmode != kRelTables) return ATTN_E_UNSUPPORTED;
  constexpr int wpe = (BIAS == ATTN_BIAS_NONE && !MASK) ? kWpeNone : 1;
  return launch_mfma<BIAS, MASK, kRelTables, wpe, 4, true>(p, a, s);
}

// HG heads of a window in one workgroup (the packed short-sequence form).
template <int HG, int BIAS, bool MASK>
int launch_winp(const Plan& p, AttnArgs a, hipStream_t s) {
  constexpr int D = INST_D;
  a.n_hgrp = a.H / HG;
  a.fd_hgrp = make_fastdiv(a.n_hgrp);
  a.n_blocks = (int)p.blocks;
  auto kern = MASK ? attn_fwd_winp<Elem, D, HG, BIAS, ATTN_MASK_SHIFT_REGIONS>
                   : attn_fwd_winp<Elem, D, HG, BIAS, ATTN_MASK_NONE>;
  return launch_grid(kern, kWinWaves * HG * 64, p, a, s);
}

template <int BIAS, bool MASK>
int launch_one(const AttnArgs& a, hipStream_t s) {
  constexpr int D = INST_D;
  const Plan p = plan_half<D>(a);
  if (p.kernel < 0 || p.lds > kMaxLds || p.blocks > 0x7fffffff) return ATTN_E_UNSUPPORTED;
  if constexpr (BIAS == ATTN_BIAS_NONE || BIAS == ATTN_BIAS_TABLE) {
    if (p.kernel == kKernWinPacked) {
      switch (p.hg) {
        case 2: return launch_winp<2, BIAS, MASK>(p, a, s);
        case 3: return launch_winp<3, BIAS, MASK>(p, a, s);
        case 4: return launch_winp<4, BIAS, MASK>(p, a, s);
        default: return ATTN_E_UNSUPPORTED;
      }
    }
  }
  if constexpr (BIAS != ATTN_BIAS_RELPOS) {
    if (a.f8) return launch_f8<BIAS, MASK>(p, a, s);
    if (p.kernel == kKernWin) return launch_win<Elem, D, BIAS, MASK>(p, a, s);
  }
  if (a.f8) return ATTN_E_UNSUPPORTED;
  if constexpr (BIAS == ATTN_BIAS_RELPOS && !MASK) {
    if (p.rmode == kRelRow64)
      return p.nw == 8 ? launch_mfma<BIAS, false, kRelRow64, 2, 8>(p, a, s)
                       : launch_mfma<BIAS, false, kRelRow64, kWpeRelpos>(p, a, s);
    if (p.rmode == kRelAug) return launch_mfma<BIAS, false, kRelAug, kWpeAug>(p, a, s);
  }
  if constexpr (BIAS == ATTN_BIAS_NONE && !MASK) {
    // Keys spanning exactly two tiles (cross-attention to short contexts):
    // both tiles are loaded with the queries, one barrier, no waits between.
    if (p.rmode == kTwoTiles)
      return launch_mfma<BIAS, MASK, kTwoTiles, two_tile_wpe<D>(), two_tile_nw<D>()>(p, a, s);
  }
  constexpr int wpe = (BIAS == ATTN_BIAS_NONE && !MASK) ? kWpeNone : 1;
  return launch_mfma<BIAS, MASK, kRelTables, wpe>(p, a, s);
}

#endif

}  // namespace

#if INST_DT != 0
// The backward launchers of this instance.
#include "attn_bwd_launch.h"
#endif

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
