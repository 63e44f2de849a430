/* A plain C11 caller of the attention library's C ABI: includes the public
 * header, links libattn.so, and checks the status attn_check returns for
 * valid calls and for each kind of argument error.  attn_check validates
 * descriptors only and never touches the device or the pointed-to memory,
 * so the tensor pointers here are distinct, 16-byte aligned addresses with
 * no memory behind them.  Exit status 0 when every check passes. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: status %d (%s), expected %d\n", what, got, attn_strerror(got), want);
    ++failures;
  }
}

/* Contiguous [B, H, N, d] tensor at a fake device address. */
static attn_tensor_t tensor(uintptr_t addr, int64_t B, int64_t H, int64_t N, int64_t d, int32_t layout) {
  attn_tensor_t t;
  memset(&t, 0, sizeof t);
  t.data = (void*)addr;
  t.dims[0] = B; t.dims[1] = H; t.dims[2] = N; t.dims[3] = d;
  t.strides[2] = d;
  t.strides[1] = N * d;
  t.strides[0] = H * N * d;
  t.layout = layout;
  return t;
}

int main(void) {
  const uintptr_t GiB = (uintptr_t)1 << 30;
  attn_tensor_t q = tensor(1 * GiB, 2, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  attn_tensor_t k = tensor(2 * GiB, 2, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  attn_tensor_t v = tensor(3 * GiB, 2, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  attn_tensor_t o = tensor(4 * GiB, 2, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  attn_bias_desc_t none_b;
  attn_mask_desc_t none_m;
  memset(&none_b, 0, sizeof none_b);
  memset(&none_m, 0, sizeof none_m);
  none_b.kind = ATTN_BIAS_NONE;
  none_m.kind = ATTN_MASK_NONE;

  expect("plain f16", attn_check(&q, &k, &v, &none_b, &none_m, &o, ATTN_F16), ATTN_OK);
  expect("plain, no descriptors", attn_check(&q, &k, &v, NULL, NULL, &o, ATTN_BF16), ATTN_OK);
  expect("NULL q", attn_check(NULL, &k, &v, NULL, NULL, &o, ATTN_F16), ATTN_E_NULL);

  attn_tensor_t k2 = tensor(2 * GiB, 1, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  expect("batch mismatch", attn_check(&q, &k2, &v, NULL, NULL, &o, ATTN_F16), ATTN_E_SHAPE);

  attn_tensor_t q48 = tensor(1 * GiB, 2, 3, 49, 48, ATTN_LAYOUT_BATCHED);
  attn_tensor_t k48 = tensor(2 * GiB, 2, 3, 49, 48, ATTN_LAYOUT_BATCHED);
  attn_tensor_t v48 = tensor(3 * GiB, 2, 3, 49, 48, ATTN_LAYOUT_BATCHED);
  attn_tensor_t o48 = tensor(4 * GiB, 2, 3, 49, 48, ATTN_LAYOUT_BATCHED);
  expect("head dim 48", attn_check(&q48, &k48, &v48, NULL, NULL, &o48, ATTN_F16), ATTN_E_UNSUPPORTED);

  attn_tensor_t qm = q;
  qm.data = (void*)(1 * GiB + 2); /* not 16-byte aligned */
  expect("misaligned q", attn_check(&qm, &k, &v, NULL, NULL, &o, ATTN_F16), ATTN_E_LAYOUT);

  attn_tensor_t oa = o;
  oa.data = q.data; /* out on top of q */
  expect("out aliases q", attn_check(&q, &k, &v, NULL, NULL, &oa, ATTN_F16), ATTN_E_ALIAS);

  expect("unknown dtype", attn_check(&q, &k, &v, NULL, NULL, &o, 9), ATTN_E_INVALID);

  /* Swin table bias on 7x7 windows with the shifted-window region mask. */
  attn_bias_desc_t tb;
  memset(&tb, 0, sizeof tb);
  tb.kind = ATTN_BIAS_TABLE;
  tb.grid_h = tb.grid_w = 7;
  tb.table = (void*)(5 * GiB);
  attn_mask_desc_t sm;
  memset(&sm, 0, sizeof sm);
  sm.kind = ATTN_MASK_SHIFT_REGIONS;
  sm.value = -100.f;
  sm.win.img_h = sm.win.img_w = 14;
  sm.win.win_h = sm.win.win_w = 7;
  sm.win.shift_h = sm.win.shift_w = 3;
  attn_tensor_t qw = tensor(1 * GiB, 8, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  attn_tensor_t kw = tensor(2 * GiB, 8, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  attn_tensor_t vw = tensor(3 * GiB, 8, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  attn_tensor_t ow = tensor(4 * GiB, 8, 3, 49, 32, ATTN_LAYOUT_BATCHED);
  expect("table + shift mask", attn_check(&qw, &kw, &vw, &tb, &sm, &ow, ATTN_F16), ATTN_OK);

  /* SAM windows from an unpadded 64x64 token image: 14x14 windows, padded to
   * 70x70 in the addressing, decomposed relative position. */
  attn_tensor_t qi = tensor(1 * GiB, 8, 12, 4096, 64, ATTN_LAYOUT_IMAGE);
  attn_tensor_t ki = tensor(2 * GiB, 8, 12, 4096, 64, ATTN_LAYOUT_IMAGE);
  attn_tensor_t vi = tensor(3 * GiB, 8, 12, 4096, 64, ATTN_LAYOUT_IMAGE);
  attn_tensor_t oi = tensor(4 * GiB, 8, 12, 4096, 64, ATTN_LAYOUT_IMAGE);
  attn_bias_desc_t rp;
  memset(&rp, 0, sizeof rp);
  rp.kind = ATTN_BIAS_RELPOS;
  rp.grid_h = rp.grid_w = 14;
  rp.rh = (void*)(5 * GiB);
  rp.rw = (void*)(6 * GiB);
  attn_mask_desc_t geo;
  memset(&geo, 0, sizeof geo);
  geo.kind = ATTN_MASK_NONE;
  geo.win.img_h = geo.win.img_w = 64;
  geo.win.win_h = geo.win.win_w = 14;
  expect("padded image relpos", attn_check(&qi, &ki, &vi, &rp, &geo, &oi, ATTN_BF16), ATTN_OK);
  geo.win.win_h = 0;
  expect("window of zero rows", attn_check(&qi, &ki, &vi, &rp, &geo, &oi, ATTN_BF16), ATTN_E_SHAPE);
  geo.win.win_h = 14;
  rp.kgrid_h = rp.kgrid_w = 7;
  expect("key grid in the image layout", attn_check(&qi, &ki, &vi, &rp, &geo, &oi, ATTN_BF16),
         ATTN_E_SHAPE);

  /* SAM global queries on the 64x64 grid against keys on a 32x32 grid: the
   * tables keep 2*64-1 rows. */
  attn_tensor_t qg = tensor(1 * GiB, 1, 12, 4096, 64, ATTN_LAYOUT_BATCHED);
  attn_tensor_t kg = tensor(2 * GiB, 1, 12, 1024, 64, ATTN_LAYOUT_BATCHED);
  attn_tensor_t vg = tensor(3 * GiB, 1, 12, 1024, 64, ATTN_LAYOUT_BATCHED);
  attn_tensor_t og = tensor(4 * GiB, 1, 12, 4096, 64, ATTN_LAYOUT_BATCHED);
  attn_bias_desc_t kgb;
  memset(&kgb, 0, sizeof kgb);
  kgb.kind = ATTN_BIAS_RELPOS;
  kgb.grid_h = kgb.grid_w = 64;
  kgb.kgrid_h = kgb.kgrid_w = 32;
  kgb.rh = (void*)(5 * GiB);
  kgb.rw = (void*)(6 * GiB);
  expect("key grid relpos", attn_check(&qg, &kg, &vg, &kgb, NULL, &og, ATTN_BF16), ATTN_OK);
  kgb.kgrid_w = 16;
  expect("key grid size mismatch", attn_check(&qg, &kg, &vg, &kgb, NULL, &og, ATTN_BF16), ATTN_E_SHAPE);

  if (attn_strerror(ATTN_E_SHAPE) == NULL || attn_strerror(12345) == NULL) {
    printf("FAIL attn_strerror returned NULL\n");
    ++failures;
  }
  if ((attn_version() >> 16) != 1) {
    printf("FAIL attn_version %d\n", attn_version());
    ++failures;
  }
  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
