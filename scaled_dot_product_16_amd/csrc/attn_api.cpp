// Host side of the C ABI: argument validation (no HIP dependency, so it can be
// exercised on a machine without a GPU through attn_check) and the exported
// entry points.  Validation ends with the call's plan (attn_plan.h: kernel
// choice and LDS bytes), so a call whose tiles or tables do not fit on chip
// is refused here, by attn_check as by attn_fwd.  The launch itself lives in
// attn_dispatch.cpp and attn_inst.hip.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/attn.h"
#include "attn_internal.h"
#include "attn_plan.h"

namespace attn {
namespace {

int elem_size(int32_t dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool head_dim_supported(int32_t dtype, int64_t d) {
  if (dtype == ATTN_F32) return d >= 4 && d <= 128 && d % 4 == 0;
  return d == 32 || d == 40 || d == 64 || d == 80;
}

// Byte range [lo, hi) touched by a strided 4-D tensor.
void extent(const attn_tensor_t* t, int es, uintptr_t* lo, uintptr_t* hi) {
  int64_t last = 0;
  for (int i = 0; i < 3; ++i) last += (t->dims[i] - 1) * t->strides[i];
  last += t->dims[3] - 1;
  *lo = (uintptr_t)t->data;
  *hi = (uintptr_t)t->data + (uintptr_t)((last + 1) * es);
}

bool overlaps(const attn_tensor_t* a, int ea, const attn_tensor_t* b, int eb) {
  uintptr_t alo, ahi, blo, bhi;
  extent(a, ea, &alo, &ahi);
  extent(b, eb, &blo, &bhi);
  return alo < bhi && blo < ahi;
}

bool overlaps(const attn_tensor_t* a, const attn_tensor_t* b, int es) { return overlaps(a, es, b, es); }

// `align`: bytes the kernels move per row piece (16; 8 for 8-bit q, k, v).
int check_tensor(const attn_tensor_t* t, int es, int align = 16) {
  if (!t->data) return ATTN_E_NULL;
  for (int i = 0; i < 4; ++i)
    if (t->dims[i] < 1 || t->dims[i] > (int64_t(1) << 30)) return ATTN_E_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (t->strides[i] < 0) return ATTN_E_LAYOUT;
  // Vector loads move `align` bytes: base and every row start must be aligned to it.
  const int64_t vec = align / es;
  if ((uintptr_t)t->data % align) return ATTN_E_LAYOUT;
  for (int i = 0; i < 3; ++i)
    if (t->strides[i] % vec) return ATTN_E_LAYOUT;
  if (t->layout != ATTN_LAYOUT_BATCHED && t->layout != ATTN_LAYOUT_IMAGE) return ATTN_E_INVALID;
  return ATTN_OK;
}

bool window_valid(const attn_window_t& w) {
  if (w.img_h < 1 || w.img_w < 1 || w.win_h < 1 || w.win_w < 1) return false;
  if (w.shift_h < 0 || w.shift_w < 0 || w.shift_h >= w.win_h || w.shift_w >= w.win_w) return false;
  if (w.img_h > kMaxGridSide * 16 || w.img_w > kMaxGridSide * 16) return false;
  if (w.win_h > kMaxGridSide || w.win_w > kMaxGridSide) return false;
  return true;
}

}  // namespace

int validate(const void* qv, const void* kv, const void* vv, const void* biasv,
             const void* maskv, const void* outv, int32_t dtype, const void* optv,
             AttnArgs* a) {
  const attn_tensor_t* q = (const attn_tensor_t*)qv;
  const attn_tensor_t* k = (const attn_tensor_t*)kv;
  const attn_tensor_t* v = (const attn_tensor_t*)vv;
  const attn_tensor_t* o = (const attn_tensor_t*)outv;
  const attn_bias_desc_t* bias = (const attn_bias_desc_t*)biasv;
  const attn_mask_desc_t* mask = (const attn_mask_desc_t*)maskv;
  if (!q || !k || !v || !o || !a) return ATTN_E_NULL;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_INVALID;
  // Options that change how q, k and v are read come first.
  const attn_options_t* opt = (const attn_options_t*)optv;
  const int32_t qkv_format = opt ? opt->qkv_format : ATTN_QKV_DTYPE;
  if (qkv_format != ATTN_QKV_DTYPE && qkv_format != ATTN_QKV_E4M3) return ATTN_E_INVALID;
  const bool f8 = qkv_format == ATTN_QKV_E4M3;
  if (f8) {
    const float sc[3] = {opt->q_descale, opt->k_descale, opt->v_descale};
    for (float x : sc)
      if (!(x > 0.f) || !isfinite(x)) return ATTN_E_INVALID;
    if (dtype == ATTN_F32) return ATTN_E_UNSUPPORTED;
  }
  if (opt && opt->window_heads < 0) return ATTN_E_INVALID;
  const int es = elem_size(dtype);
  const int ies = f8 ? 1 : es;  // bytes of a q, k or v element
  const int ialign = f8 ? 8 : 16;
  int st;
  if ((st = check_tensor(q, ies, ialign)) || (st = check_tensor(k, ies, ialign)) ||
      (st = check_tensor(v, ies, ialign)) || (st = check_tensor(o, es)))
    return st;

  // Shapes: [B, H, N, d] with shared B, H, d; k and v share N; out matches q.
  const int64_t B = q->dims[0], H = q->dims[1], Nq = q->dims[2], D = q->dims[3];
  const int64_t Nk = k->dims[2];
  if (k->dims[0] != B || v->dims[0] != B || o->dims[0] != B) return ATTN_E_SHAPE;
  if (k->dims[1] != H || v->dims[1] != H || o->dims[1] != H) return ATTN_E_SHAPE;
  if (k->dims[3] != D || v->dims[3] != D || o->dims[3] != D) return ATTN_E_SHAPE;
  if (v->dims[2] != Nk || o->dims[2] != Nq) return ATTN_E_SHAPE;
  if (!head_dim_supported(dtype, D)) return ATTN_E_UNSUPPORTED;

  const int32_t layout = q->layout;
  if (k->layout != layout || v->layout != layout || o->layout != layout) return ATTN_E_LAYOUT;

  const int32_t bias_kind = bias ? bias->kind : ATTN_BIAS_NONE;
  const int32_t mask_kind = mask ? mask->kind : ATTN_MASK_NONE;
  if (bias_kind < ATTN_BIAS_NONE || bias_kind > ATTN_BIAS_ADDITIVE) return ATTN_E_INVALID;
  if (mask_kind < ATTN_MASK_NONE || mask_kind > ATTN_MASK_SHIFT_REGIONS) return ATTN_E_INVALID;

  memset(a, 0, sizeof(*a));
  a->q = q->data;
  a->k = k->data;
  a->v = v->data;
  a->o = o->data;
  a->q_sb = q->strides[0]; a->q_sh = q->strides[1]; a->q_sn = q->strides[2];
  a->k_sb = k->strides[0]; a->k_sh = k->strides[1]; a->k_sn = k->strides[2];
  a->v_sb = v->strides[0]; a->v_sh = v->strides[1]; a->v_sn = v->strides[2];
  a->o_sb = o->strides[0]; a->o_sh = o->strides[1]; a->o_sn = o->strides[2];
  a->dtype = dtype;
  a->H = (int32_t)H;
  a->D = (int32_t)D;
  a->scale = (float)(1.0 / sqrt((double)D));
  if (f8) {
    // q and k scales multiply every score, so they join the softmax scale.
    a->f8 = 1;
    a->scale = (float)((double)opt->q_descale * (double)opt->k_descale / sqrt((double)D));
    a->v_descale = opt->v_descale;
    if (!(a->scale > 0.f) || !isfinite(a->scale)) return ATTN_E_INVALID;
  }

  // Window geometry: needed by IMAGE layout and by SHIFT_REGIONS.
  const bool need_win = layout == ATTN_LAYOUT_IMAGE || mask_kind == ATTN_MASK_SHIFT_REGIONS;
  int64_t Beff = B, nq_eff = Nq, nk_eff = Nk;
  if (need_win) {
    if (!mask) return ATTN_E_NULL;
    const attn_window_t& w = mask->win;
    if (!window_valid(w)) return ATTN_E_SHAPE;
    a->img_h = w.img_h; a->img_w = w.img_w; a->win_h = w.win_h; a->win_w = w.win_w;
    a->shift_h = w.shift_h; a->shift_w = w.shift_w;
    // Zero padding at the bottom and right up to whole windows.
    a->pimg_h = (w.img_h + w.win_h - 1) / w.win_h * w.win_h;
    a->pimg_w = (w.img_w + w.win_w - 1) / w.win_w * w.win_w;
    a->nwx = a->pimg_w / w.win_w;
    a->nw = (a->pimg_h / w.win_h) * a->nwx;
    const int64_t wt = (int64_t)w.win_h * w.win_w;
    if (layout == ATTN_LAYOUT_IMAGE) {
      if (Nq != (int64_t)w.img_h * w.img_w || Nk != Nq) return ATTN_E_SHAPE;
      a->image = 1;
      Beff = B * a->nw;
      nq_eff = nk_eff = wt;
    } else if (Nq != wt || Nk != wt) {
      return ATTN_E_SHAPE;
    }
  }
  if (Beff > (int64_t(1) << 30)) return ATTN_E_UNSUPPORTED;
  a->B = (int32_t)Beff;
  a->Nq = (int32_t)nq_eff;
  a->Nk = (int32_t)nk_eff;

  // Bias.
  a->bias_kind = bias_kind;
  if (bias && bias_kind != ATTN_BIAS_RELPOS && (bias->rh_rows != 0 || bias->rw_rows != 0))
    return ATTN_E_SHAPE;  // stored table lengths belong to the relative position
  if (bias_kind == ATTN_BIAS_TABLE || bias_kind == ATTN_BIAS_RELPOS) {
    if (bias->grid_h < 1 || bias->grid_w < 1) return ATTN_E_SHAPE;
    if (bias->grid_h > kMaxGridSide || bias->grid_w > kMaxGridSide) return ATTN_E_UNSUPPORTED;
    // Keys on a grid of their own: relative position, batched layout only.
    int32_t kgh = bias->grid_h, kgw = bias->grid_w;
    if (bias->kgrid_h != 0 || bias->kgrid_w != 0) {
      if (bias_kind != ATTN_BIAS_RELPOS || a->image) return ATTN_E_SHAPE;
      if (bias->kgrid_h < 1 || bias->kgrid_w < 1) return ATTN_E_SHAPE;
      if (bias->kgrid_h > kMaxGridSide || bias->kgrid_w > kMaxGridSide) return ATTN_E_UNSUPPORTED;
      kgh = bias->kgrid_h;
      kgw = bias->kgrid_w;
    }
    const int64_t g = (int64_t)bias->grid_h * bias->grid_w;
    const int64_t kg = (int64_t)kgh * kgw;
    if (nq_eff != g || nk_eff != kg) return ATTN_E_SHAPE;
    if (g > kMaxIndexedTokens || kg > kMaxIndexedTokens) return ATTN_E_UNSUPPORTED;
    a->gh = bias->grid_h;
    a->gw = bias->grid_w;
    a->kgh = kgh;
    a->kgw = kgw;
    if (bias_kind == ATTN_BIAS_TABLE) {
      if (!bias->table) return ATTN_E_NULL;
      if ((int64_t)(2 * a->gh - 1) * (2 * a->gw - 1) > 16384) return ATTN_E_UNSUPPORTED;
      a->table = bias->table;
    } else {
      if (!bias->rh || !bias->rw) return ATTN_E_NULL;
      if ((uintptr_t)bias->rh % 16 || (uintptr_t)bias->rw % 16) return ATTN_E_LAYOUT;
      // Table rows per axis: 2 * max(query, key positions) - 1.
      if ((a->gh > a->kgh ? a->gh : a->kgh) + (a->gw > a->kgw ? a->gw : a->kgw) > 256)
        return ATTN_E_UNSUPPORTED;
      // Stored rows (0: the rows needed); another length is resized in the
      // kernel.
      if (bias->rh_rows < 0 || bias->rw_rows < 0) return ATTN_E_SHAPE;
      if (bias->rh_rows > 1023 || bias->rw_rows > 1023) return ATTN_E_UNSUPPORTED;
      a->rh_rows = bias->rh_rows ? bias->rh_rows : 2 * (a->gh > a->kgh ? a->gh : a->kgh) - 1;
      a->rw_rows = bias->rw_rows ? bias->rw_rows : 2 * (a->gw > a->kgw ? a->gw : a->kgw) - 1;
      a->rh = bias->rh;
      a->rw = bias->rw;
    }
  } else if (bias_kind == ATTN_BIAS_ADDITIVE) {
    if (!bias->add) return ATTN_E_NULL;
    if (bias->add_batch < 1 || bias->add_strides[0] < 0 || bias->add_strides[1] < 0)
      return ATTN_E_SHAPE;
    a->badd = bias->add;
    a->badd_n = bias->add_batch;
    a->badd_s0 = bias->add_strides[0];
    a->badd_s1 = bias->add_strides[1];
  }

  // Mask.
  a->mask_kind = mask_kind;
  if (mask_kind == ATTN_MASK_SHIFT_REGIONS) {
    if (nq_eff > kMaxIndexedTokens) return ATTN_E_UNSUPPORTED;
    if (!isfinite(mask->value)) return ATTN_E_INVALID;
    a->mask_value = mask->value;
  } else if (mask_kind == ATTN_MASK_ADDITIVE) {
    if (!mask->add) return ATTN_E_NULL;
    if (mask->n_win < 1 || mask->add_strides[0] < 0 || mask->add_strides[1] < 0)
      return ATTN_E_SHAPE;
    a->madd = mask->add;
    a->madd_n = mask->n_win;
    a->madd_s0 = mask->add_strides[0];
    a->madd_s1 = mask->add_strides[1];
  }

  a->fd_h = make_fastdiv(a->H);
  a->fd_nw = make_fastdiv(a->nw);
  a->fd_nwx = make_fastdiv(a->nwx);
  a->fd_win_w = make_fastdiv(a->win_w);
  a->fd_gw = make_fastdiv(a->gw);
  a->fd_kgw = make_fastdiv(a->kgw);

  // Offsets inside one (batch item, head) slice are 32-bit in the kernels.
  const attn_tensor_t* ts[4] = {q, k, v, o};
  // Image layout: below 2^29, so that byte offsets of 16-bit and 32-bit
  // elements stay clear of the padding-token marker.
  const int slice_bits = a->image ? 29 : 31;
  for (const attn_tensor_t* t : ts)
    if ((t->dims[2] - 1) * t->strides[2] + t->dims[3] >= (int64_t(1) << slice_bits)) return ATTN_E_UNSUPPORTED;

  // out must not overlap the inputs it is computed from.
  if (overlaps(o, es, q, ies) || overlaps(o, es, k, ies) || overlaps(o, es, v, ies)) return ATTN_E_ALIAS;

  if (opt) a->win_heads = opt->window_heads;
  if (opt && opt->lse) {
    // Per-row log-sum-exp: [B, H, N] fp32 (N: the tokens of q's layout).
    if (dtype == ATTN_F32) return ATTN_E_UNSUPPORTED;
    if ((uintptr_t)opt->lse % 4) return ATTN_E_LAYOUT;
    attn_tensor_t lt{};
    lt.data = opt->lse;
    lt.dims[0] = q->dims[0]; lt.dims[1] = q->dims[1]; lt.dims[2] = q->dims[2]; lt.dims[3] = 1;
    lt.strides[2] = 1; lt.strides[1] = q->dims[2]; lt.strides[0] = q->dims[1] * q->dims[2];
    if (overlaps(&lt, 4, o, es) || overlaps(&lt, 4, q, ies) || overlaps(&lt, 4, k, ies) ||
        overlaps(&lt, 4, v, ies))
      return ATTN_E_ALIAS;
    a->lse = opt->lse;
  }

  // The kernel the call takes must fit one CU's LDS (and the grid the
  // launch limit); a requested form must exist for the call.
  Plan plan;
  return make_plan(*a, &plan);
}

int validate_bwd(const void* qv, const void* kv, const void* vv, const void* dov, const void* biasv,
                 const void* maskv, const void* dqv, const void* dkv, const void* dvv, float* dtable,
                 int32_t dtype, AttnBwdArgs* ba, size_t* ws_bytes, const void* optv) {
  if (!ba || !ws_bytes) return ATTN_E_NULL;
  memset(ba, 0, sizeof(*ba));
  *ws_bytes = 0;
  // The forward validation, with dO in the place of the output.
  int st = validate(qv, kv, vv, biasv, maskv, dov, dtype, nullptr, &ba->a);
  if (st != ATTN_OK) return st;
  const attn_tensor_t* q = (const attn_tensor_t*)qv;
  const attn_tensor_t* k = (const attn_tensor_t*)kv;
  const attn_tensor_t* v = (const attn_tensor_t*)vv;
  const attn_tensor_t* dout = (const attn_tensor_t*)dov;
  const attn_tensor_t* dq = (const attn_tensor_t*)dqv;
  const attn_tensor_t* dk = (const attn_tensor_t*)dkv;
  const attn_tensor_t* dv = (const attn_tensor_t*)dvv;
  if (!dq || !dk || !dv) return ATTN_E_NULL;
  const int es = elem_size(dtype);
  if ((st = check_tensor(dq, es)) || (st = check_tensor(dk, es)) || (st = check_tensor(dv, es))) return st;
  const attn_tensor_t* pairs[3][2] = {{dq, q}, {dk, k}, {dv, v}};
  for (auto& pr : pairs) {
    for (int i = 0; i < 4; ++i)
      if (pr[0]->dims[i] != pr[1]->dims[i]) return ATTN_E_SHAPE;
    if (pr[0]->layout != pr[1]->layout) return ATTN_E_LAYOUT;
    const int slice_bits = ba->a.image ? 29 : 31;
    if ((pr[0]->dims[2] - 1) * pr[0]->strides[2] + pr[0]->dims[3] >= (int64_t(1) << slice_bits))
      return ATTN_E_UNSUPPORTED;
  }
  // Gradients overlap neither the inputs nor each other.
  const attn_tensor_t* ins[4] = {q, k, v, dout};
  const attn_tensor_t* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (const attn_tensor_t* t : ins)
      if (overlaps(outs[i], t, es)) return ATTN_E_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j], es)) return ATTN_E_ALIAS;
  }
  // Built (the backward plan): window units (at most 64 queries and keys,
  // any bias but the relative position, any mask), and the tiled path for
  // longer sequences with no bias or the relative position (equal grids,
  // tables of the needed length), no mask, batched layout.
  Plan plan;
  if ((st = make_bwd_plan(ba->a, &plan)) != ATTN_OK) return st;
  ba->dq = dq->data;
  ba->dk = dk->data;
  ba->dv = dv->data;
  ba->dq_sb = dq->strides[0]; ba->dq_sh = dq->strides[1]; ba->dq_sn = dq->strides[2];
  ba->dk_sb = dk->strides[0]; ba->dk_sh = dk->strides[1]; ba->dk_sn = dk->strides[2];
  ba->dv_sb = dv->strides[0]; ba->dv_sh = dv->strides[1]; ba->dv_sn = dv->strides[2];
  if (ba->a.bias_kind == ATTN_BIAS_TABLE || ba->a.bias_kind == ATTN_BIAS_RELPOS) {
    // TABLE: [(2gh-1)(2gw-1), H]; RELPOS: the stacked [dRh; dRw] rows of d.
    if (!dtable) return ATTN_E_NULL;
    if ((uintptr_t)dtable % 4) return ATTN_E_LAYOUT;
    ba->n_tab = ba->a.bias_kind == ATTN_BIAS_TABLE ? (2 * ba->a.gh - 1) * (2 * ba->a.gw - 1)
                                                   : bwd_rel_rows(ba->a);
    ba->dtable = dtable;
  }
  // The forward's O and log-sum-exp (attn_bwd_opt): O shaped and laid out
  // like dout, lse [B, H, Nq] fp32; neither may overlap a gradient.
  const attn_bwd_options_t* opt = (const attn_bwd_options_t*)optv;
  if (opt && (opt->out || opt->lse)) {
    if (!opt->out || !opt->lse) return ATTN_E_NULL;
    const attn_tensor_t* fo = opt->out;
    if ((st = check_tensor(fo, es)) != ATTN_OK) return st;
    for (int i = 0; i < 4; ++i)
      if (fo->dims[i] != dout->dims[i]) return ATTN_E_SHAPE;
    if (fo->layout != dout->layout) return ATTN_E_LAYOUT;
    if ((fo->dims[2] - 1) * fo->strides[2] + fo->dims[3] >= (int64_t(1) << (ba->a.image ? 29 : 31)))
      return ATTN_E_UNSUPPORTED;
    if ((uintptr_t)opt->lse % 4) return ATTN_E_LAYOUT;
    attn_tensor_t lt{};
    lt.data = (void*)opt->lse;
    lt.dims[0] = q->dims[0]; lt.dims[1] = q->dims[1]; lt.dims[2] = q->dims[2]; lt.dims[3] = 1;
    lt.strides[2] = 1; lt.strides[1] = q->dims[2]; lt.strides[0] = q->dims[1] * q->dims[2];
    for (int i = 0; i < 3; ++i)
      if (overlaps(outs[i], fo, es) || overlaps(outs[i], es, &lt, 4)) return ATTN_E_ALIAS;
    ba->fo = fo->data;
    ba->fo_sb = fo->strides[0]; ba->fo_sh = fo->strides[1]; ba->fo_sn = fo->strides[2];
    ba->lse_in = opt->lse;
  }
  *ws_bytes = bwd_workspace_bytes(ba->a, plan.kernel);
  return ATTN_OK;
}

namespace {

int check_workspace(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return ATTN_OK;
  if (!ws) return ATTN_E_NULL;
  if ((uintptr_t)ws % 16) return ATTN_E_LAYOUT;
  if (ws_bytes < need) return ATTN_E_SHAPE;
  return ATTN_OK;
}

}  // namespace

}  // namespace attn

extern "C" {

int attn_bwd_workspace_size(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                            const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
                            const attn_mask_desc_t* mask_desc, int32_t dtype, size_t* bytes) {
  if (!bytes) return ATTN_E_NULL;
  *bytes = 0;
  attn::AttnArgs a;
  int st = attn::validate(q, k, v, bias_desc, mask_desc, dout, dtype, nullptr, &a);
  if (st != ATTN_OK) return st;
  attn::Plan plan;
  if ((st = attn::make_bwd_plan(a, &plan)) != ATTN_OK) return st;
  *bytes = attn::bwd_workspace_bytes(a, plan.kernel);
  return ATTN_OK;
}

int attn_bwd_check(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                   const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
                   const attn_mask_desc_t* mask_desc, const attn_tensor_t* dq, const attn_tensor_t* dk,
                   const attn_tensor_t* dv, float* dtable, int32_t dtype, void* workspace,
                   size_t workspace_bytes) {
  attn::AttnBwdArgs ba;
  size_t need = 0;
  int st = attn::validate_bwd(q, k, v, dout, bias_desc, mask_desc, dq, dk, dv, dtable, dtype, &ba, &need,
                              nullptr);
  if (st != ATTN_OK) return st;
  return attn::check_workspace(workspace, workspace_bytes, need);
}

int attn_bwd_opt(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                 const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
                 const attn_mask_desc_t* mask_desc, const attn_tensor_t* dq, const attn_tensor_t* dk,
                 const attn_tensor_t* dv, float* dtable, int32_t dtype,
                 const attn_bwd_options_t* options, void* workspace, size_t workspace_bytes,
                 void* stream) {
  attn::AttnBwdArgs ba;
  size_t need = 0;
  int st = attn::validate_bwd(q, k, v, dout, bias_desc, mask_desc, dq, dk, dv, dtable, dtype, &ba, &need,
                              options);
  if (st != ATTN_OK) return st;
  if ((st = attn::check_workspace(workspace, workspace_bytes, need)) != ATTN_OK) return st;
  ba.ws = (float*)workspace;
  return attn::launch_bwd(ba, stream);
}

int attn_bwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
             const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
             const attn_mask_desc_t* mask_desc, const attn_tensor_t* dq, const attn_tensor_t* dk,
             const attn_tensor_t* dv, float* dtable, int32_t dtype, void* workspace,
             size_t workspace_bytes, void* stream) {
  return attn_bwd_opt(q, k, v, dout, bias_desc, mask_desc, dq, dk, dv, dtable, dtype, nullptr, workspace,
                      workspace_bytes, stream);
}

int attn_check_opt(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                   const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
                   const attn_tensor_t* out, int32_t dtype, const attn_options_t* options) {
  attn::AttnArgs a;
  return attn::validate(q, k, v, bias_desc, mask_desc, out, dtype, options, &a);
}

int attn_fwd_opt(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                 const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
                 const attn_tensor_t* out, int32_t dtype, const attn_options_t* options,
                 void* stream) {
  attn::AttnArgs a;
  int st = attn::validate(q, k, v, bias_desc, mask_desc, out, dtype, options, &a);
  if (st != ATTN_OK) return st;
  return attn::launch(a, stream);
}

int attn_check(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
               const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
               const attn_tensor_t* out, int32_t dtype) {
  return attn_check_opt(q, k, v, bias_desc, mask_desc, out, dtype, nullptr);
}

int attn_fwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
             const attn_bias_desc_t* bias_desc, const attn_mask_desc_t* mask_desc,
             const attn_tensor_t* out, int32_t dtype, void* stream) {
  return attn_fwd_opt(q, k, v, bias_desc, mask_desc, out, dtype, nullptr, stream);
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "inconsistent shapes, grid or window geometry";
    case ATTN_E_LAYOUT: return "unsupported strides, layout or alignment";
    case ATTN_E_UNSUPPORTED: return "head dim, dtype or size not supported";
    case ATTN_E_ALIAS: return "out overlaps q, k or v";
    case ATTN_E_LAUNCH: return "kernel launch failed";
    case ATTN_E_INVALID: return "invalid enum value or field";
    default: return "unknown status";
  }
}

int attn_version(void) { return (1 << 16) | 5; }

}  // extern "C"
