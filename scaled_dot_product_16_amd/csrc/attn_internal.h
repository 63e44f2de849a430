// Internal interface between the host validation layer (attn_api.cpp, no HIP
// dependency) and the kernel launcher (attn_dispatch.cpp, attn_inst.hip).
#ifndef ATTN_INTERNAL_H_
#define ATTN_INTERNAL_H_

#include <stdint.h>

namespace attn {

// Division by a runtime constant d >= 1 as a multiply-high, an add and a
// shift: n / d == (mulhi(n, mul) + n) >> shift for 0 <= n < 2^31, with
// shift = ceil(log2 d) and mul = floor(2^(32+shift) / d) + 1 - 2^32.
struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

inline FastDiv make_fastdiv(int64_t d) {
  if (d < 1) d = 1;
  uint32_t s = 0;
  while ((int64_t(1) << s) < d) ++s;
  const unsigned __int128 m = ((unsigned __int128)1 << (32 + s)) / (uint64_t)d + 1;
  return FastDiv{(uint32_t)(uint64_t)(m - ((unsigned __int128)1 << 32)), s};
}

// A validated call, flattened into plain integers and pointers.  Passed by
// value to every kernel, so it must stay trivially copyable.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int32_t dtype;
  int32_t B;     // batch items as attention sees them (images * windows for IMAGE)
  int32_t H;
  int32_t Nq;    // tokens per batch item (window tokens for IMAGE)
  int32_t Nk;
  int32_t D;
  // Window geometry (IMAGE layout address folding and SHIFT_REGIONS labels).
  int32_t image;
  int32_t img_h, img_w, win_h, win_w, shift_h, shift_w;
  int32_t pimg_h, pimg_w;  // image padded to whole windows
  int32_t nwx, nw;
  // Bias.
  int32_t bias_kind;
  int32_t gh, gw;    // grid of the queries (TABLE, RELPOS)
  int32_t kgh, kgw;  // grid of the keys (== gh, gw except for RELPOS with a key grid)
  int32_t rh_rows, rw_rows;  // RELPOS: rows stored in Rh, Rw (resized in the kernel when
                             // they differ from 2*max(gh, kgh)-1, 2*max(gw, kgw)-1)
  const void* table;
  const void* rh;
  const void* rw;
  const void* badd;
  int64_t badd_n, badd_s0, badd_s1;
  // Mask.
  int32_t mask_kind;
  const void* madd;
  int64_t madd_n, madd_s0, madd_s1;
  float mask_value;
  float scale;
  // Divisors used in index arithmetic.
  FastDiv fd_h, fd_nw, fd_nwx, fd_win_w, fd_gw, fd_kgw, fd_qt;
  // Filled by the launcher.
  int32_t n_qtiles;
  int32_t n_blocks;  // workgroups in the grid
  int32_t tpw;       // two-tile form, batched layout: consecutive query tiles per workgroup (0: one)
  int32_t n_hgrp;    // head groups per batch item (packed window kernel)
  FastDiv fd_hgrp;
  int32_t win_heads; // requested heads per workgroup of the window path (0: library's choice)
  int32_t f8;        // q, k, v are E4M3 codes (their q and k scales are folded into `scale`)
  float v_descale;   // E4M3 inputs: the scale of v, applied with the row-sum division
  float* lse;        // per-row log-sum-exp output (natural log), or null
};

// A validated backward call: the forward call (its `o` is the output
// gradient dO) and the gradient outputs.
struct AttnBwdArgs {
  AttnArgs a;
  void* dq;
  void* dk;
  void* dv;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  float* dtable;  // [n_tab, H] (TABLE bias), [n_tab, D] (RELPOS: [dRh; dRw]) or null
  float* ws;      // workspace: per-window table gradients [H][n_tab][B], or the tiled path's
  int32_t n_tab;  // table rows (TABLE bias, RELPOS), else 0
  // The forward's output O and per-row log-sum-exp (attn_bwd_opt), or null.
  const void* fo;
  int64_t fo_sb, fo_sh, fo_sn;
  const float* lse_in;
};

// Host-side validation shared by attn_check and attn_fwd.  Returns an ATTN_*
// status and fills *a on success.
int validate(const void* q, const void* k, const void* v, const void* bias_desc,
             const void* mask_desc, const void* out, int32_t dtype, const void* options,
             AttnArgs* a);

// Queue the kernel for a validated call on `stream` (a hipStream_t).
int launch(const AttnArgs& a, void* stream);

// Validation of a backward call; fills *ba (and *ws_bytes, the workspace the
// call needs) on success.
int validate_bwd(const void* q, const void* k, const void* v, const void* dout, const void* bias_desc,
                 const void* mask_desc, const void* dq, const void* dk, const void* dv, float* dtable,
                 int32_t dtype, AttnBwdArgs* ba, size_t* ws_bytes, const void* bwd_options);

// Queue the backward kernels of a validated call.
int launch_bwd(const AttnBwdArgs& ba, void* stream);

// Largest grid side accepted for TABLE/RELPOS/SHIFT_REGIONS and the largest
// token count of a batch item for which per-key index data fits on chip.
constexpr int kMaxGridSide = 1024;

constexpr int kMaxIndexedTokens = 16384;

// Token offset that marks a padding token of the image layout (no memory
// behind it: loads give zero, stores are skipped).
constexpr uint32_t kPadTok = 0xFFFFFFFFu;

}  // namespace attn

#endif  // ATTN_INTERNAL_H_
