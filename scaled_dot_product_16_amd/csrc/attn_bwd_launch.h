// Launchers of the backward kernels for one compiled instance: included by
// attn_inst.hip inside namespace attn, for half precision (INST_DT != 0),
// with its Elem (the element type) and INST_D (the head dim).  The kernels
// and their form come from the call's backward plan (attn_plan_bwd.h).
#ifndef ATTN_BWD_LAUNCH_H_
#define ATTN_BWD_LAUNCH_H_

namespace {

// Backward of window units, then (table bias) the reduction of the per-unit
// table gradients.
template <int BIAS, int MASKK>
int launch_bwd_one(const AttnBwdArgs& ba0, const Plan& p, hipStream_t s) {
  AttnBwdArgs ba = ba0;
  ba.a.n_qtiles = 1;
  ba.a.fd_qt = make_fastdiv(1);
  ba.a.n_blocks = (int)p.blocks;
  auto kern = attn_bwd_win<Elem, INST_D, BIAS, MASKK>;
  if (p.lds > 32 * 1024 &&
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds) !=
          hipSuccess)
    return ATTN_E_LAUNCH;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.blocks), dim3(kWinWaves * 64), p.lds, s, ba);
  if (hipGetLastError() != hipSuccess) return ATTN_E_LAUNCH;
  if constexpr (BIAS == ATTN_BIAS_TABLE) {
    const int n = ba.n_tab * ba.a.H;
    hipLaunchKernelGGL(attn_bwd_table_reduce<0>, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, (const float*)ba.ws,
                       ba.dtable, ba.a.B, ba.a.H, ba.n_tab);
    if (hipGetLastError() != hipSuccess) return ATTN_E_LAUNCH;
  }
  return ATTN_OK;
}

template <int BIAS>
int launch_bwd_bias(const AttnBwdArgs& ba, const Plan& p, hipStream_t s) {
  switch (ba.a.mask_kind) {
    case ATTN_MASK_NONE: return launch_bwd_one<BIAS, ATTN_MASK_NONE>(ba, p, s);
    case ATTN_MASK_ADDITIVE: return launch_bwd_one<BIAS, ATTN_MASK_ADDITIVE>(ba, p, s);
    default: return launch_bwd_one<BIAS, ATTN_MASK_SHIFT_REGIONS>(ba, p, s);
  }
}
}  // namespace

// Long sequences: the row kernel (L, D, dQ), then the column kernel (dK, dV).
template <int RP>
static int launch_bwd_tiled_rp(const AttnBwdArgs& ba0, const Plan& p, hipStream_t s) {
  constexpr int D = INST_D;
  AttnBwdArgs ba = ba0;
  // Two 16-query (16-key) blocks per row (column) kernel wave where no bias
  // term is staged (up to d = 64: at d = 80 the accumulators exceed 256
  // registers).
  constexpr int KB = RP == kBwdRelNone && D <= 64 ? 2 : 1;
  ba.a.n_qtiles = (ba.a.Nq + 64 * KB - 1) / (64 * KB);  // query tiles (64 KB queries) of the row kernel
  ba.a.fd_qt = make_fastdiv(ba.a.n_qtiles);
  ba.a.n_blocks = ba.a.n_qtiles * ba.a.H * ba.a.B;
  const int n_row_wg = ba.a.n_blocks;
  auto rows = attn_bwd_rows<Elem, D, RP, KB>;
  auto cols = attn_bwd_cols<Elem, D, RP, KB>;
  if (p.lds > 32 * 1024 &&
      (hipFuncSetAttribute((const void*)rows, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds) !=
           hipSuccess ||
       hipFuncSetAttribute((const void*)cols, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds) !=
           hipSuccess))
    return ATTN_E_LAUNCH;
  hipLaunchKernelGGL(rows, dim3((unsigned)ba.a.n_blocks), dim3(256), p.lds, s, ba);
  if (hipGetLastError() != hipSuccess) return ATTN_E_LAUNCH;
  ba.a.n_qtiles = (ba.a.Nk + 64 * KB - 1) / (64 * KB);  // key tiles (64 KB keys) of the column kernel
  ba.a.fd_qt = make_fastdiv(ba.a.n_qtiles);
  ba.a.n_blocks = ba.a.n_qtiles * ba.a.H * ba.a.B;
  hipLaunchKernelGGL(cols, dim3((unsigned)ba.a.n_blocks), dim3(256), p.lds, s, ba);
  if (hipGetLastError() != hipSuccess) return ATTN_E_LAUNCH;
  if constexpr (RP != kBwdRelNone) {
    // [dRh; dRw] = fixed-order sum of the row kernel's per-workgroup parts,
    // in S slices when the table alone would leave the chip idle; the slice
    // sums go to the workspace's L and D rows (dead once the column kernel
    // is done), which must hold S * n_out floats.
    const int n_out = bwd_rel_rows(ba.a) * D;
    const int chunks = (n_out + 63) / 64;
    const int64_t room = 2 * (int64_t)ba.a.B * ba.a.H * ba.a.Nq / n_out;
    int S = (512 + chunks - 1) / chunks;
    S = (int)(S < 16 ? S : 16);
    S = (int)(S < room ? S : room);
    S = S < n_row_wg ? S : n_row_wg;
    S = S > 1 ? S : 1;
    const BwdWs wl = bwd_ws_layout(ba.a);
    float* sums = S > 1 ? ba.ws + wl.L : ba.dtable;
    hipLaunchKernelGGL(attn_bwd_part_reduce<0>, dim3((unsigned)chunks, (unsigned)S), dim3(1024), 0, s,
                       (const float*)(ba.ws + wl.part), sums, n_out, n_row_wg, (int64_t)wl.pstride, S);
    if (hipGetLastError() != hipSuccess) return ATTN_E_LAUNCH;
    if (S > 1) {
      hipLaunchKernelGGL(attn_bwd_part_final<0>, dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, s,
                         (const float*)sums, ba.dtable, n_out, S);
      if (hipGetLastError() != hipSuccess) return ATTN_E_LAUNCH;
    }
  }
  return ATTN_OK;
}

static int launch_bwd_tiled(const AttnBwdArgs& ba, const Plan& p, hipStream_t s) {
  switch (p.rmode) {
    case kBwdRelNone: return launch_bwd_tiled_rp<kBwdRelNone>(ba, p, s);
    case kBwdRelGeneral: return launch_bwd_tiled_rp<kBwdRelGeneral>(ba, p, s);
    case kBwdRelRow64: return launch_bwd_tiled_rp<kBwdRelRow64>(ba, p, s);
    case kBwdRelAug: return launch_bwd_tiled_rp<kBwdRelAug>(ba, p, s);
    default: return ATTN_E_UNSUPPORTED;
  }
}

template <>
int launch_bwd_inst<INST_DT, INST_D>(const AttnBwdArgs& ba, void* stream) {
  Plan p;
  const int st = make_bwd_plan(ba.a, &p);
  if (st != ATTN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (p.kernel == kKernMfma) return launch_bwd_tiled(ba, p, s);
  switch (ba.a.bias_kind) {
    case ATTN_BIAS_NONE: return launch_bwd_bias<ATTN_BIAS_NONE>(ba, p, s);
    case ATTN_BIAS_TABLE: return launch_bwd_bias<ATTN_BIAS_TABLE>(ba, p, s);
    case ATTN_BIAS_ADDITIVE: return launch_bwd_bias<ATTN_BIAS_ADDITIVE>(ba, p, s);
    default: return ATTN_E_UNSUPPORTED;
  }
}

#endif  // ATTN_BWD_LAUNCH_H_
