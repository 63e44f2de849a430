/* A plain C11 caller of attn_fwd on the GPU: device buffers from hipMalloc,
 * the call queued on a HIP stream, results copied back and checked against
 * closed forms of the attention definition (no oracle needed):
 *   1. one key (Nk = 1): every output row equals that key's value row,
 *      bit for bit (the softmax over one key is exactly 1);
 *   2. every value row the same vector c: every output row equals c (the
 *      probabilities sum to one), within the fp32 tolerance 1e-5 (values up
 *      to 5 in magnitude, 50 keys: a few ulps of rounding in the sums).
 * Exit status 0 when both hold; prints what failed otherwise. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attn.h"

#define HIP_OK(x)                                                   \
  do {                                                              \
    hipError_t e_ = (x);                                            \
    if (e_ != hipSuccess) {                                         \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                      \
    }                                                               \
  } while (0)

static attn_tensor_t tensor(void* p, int64_t B, int64_t H, int64_t N, int64_t d) {
  attn_tensor_t t;
  memset(&t, 0, sizeof t);
  t.data = p;
  t.dims[0] = B; t.dims[1] = H; t.dims[2] = N; t.dims[3] = d;
  t.strides[2] = d; t.strides[1] = N * d; t.strides[0] = H * N * d;
  t.layout = ATTN_LAYOUT_BATCHED;
  return t;
}

/* Deterministic values in [-2, 2) (a 32-bit LCG). */
static uint32_t lcg = 12345u;
static float next_val(void) {
  lcg = lcg * 1664525u + 1013904223u;
  return (float)(lcg >> 8) / (float)(1u << 24) * 4.f - 2.f;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static int case_single_key(hipStream_t s) {
  const int B = 2, H = 3, Nq = 130, Nk = 1, d = 64;
  const size_t nq = (size_t)B * H * Nq * d, nk = (size_t)B * H * Nk * d;
  uint16_t* hq = malloc(nq * 2); uint16_t* hk = malloc(nk * 2);
  uint16_t* hv = malloc(nk * 2); uint16_t* ho = malloc(nq * 2);
  for (size_t i = 0; i < nq; ++i) hq[i] = to_bf16(next_val());
  for (size_t i = 0; i < nk; ++i) { hk[i] = to_bf16(next_val()); hv[i] = to_bf16(next_val()); }
  void *dq, *dk, *dv, *dout;
  HIP_OK(hipMalloc(&dq, nq * 2)); HIP_OK(hipMalloc(&dk, nk * 2));
  HIP_OK(hipMalloc(&dv, nk * 2)); HIP_OK(hipMalloc(&dout, nq * 2));
  HIP_OK(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, hk, nk * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, hv, nk * 2, hipMemcpyHostToDevice));
  attn_tensor_t q = tensor(dq, B, H, Nq, d), k = tensor(dk, B, H, Nk, d);
  attn_tensor_t v = tensor(dv, B, H, Nk, d), o = tensor(dout, B, H, Nq, d);
  int st = attn_fwd(&q, &k, &v, NULL, NULL, &o, ATTN_BF16, s);
  if (st != ATTN_OK) { printf("FAIL single key: attn_fwd %s\n", attn_strerror(st)); return 1; }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(ho, dout, nq * 2, hipMemcpyDeviceToHost));
  int bad = 0;
  for (int bh = 0; bh < B * H; ++bh)
    for (int i = 0; i < Nq; ++i)
      for (int c = 0; c < d; ++c)
        if (ho[((size_t)bh * Nq + i) * d + c] != hv[(size_t)bh * d + c]) ++bad;
  if (bad) printf("FAIL single key: %d outputs differ from v row 0\n", bad);
  HIP_OK(hipFree(dq)); HIP_OK(hipFree(dk)); HIP_OK(hipFree(dv)); HIP_OK(hipFree(dout));
  free(hq); free(hk); free(hv); free(ho);
  return bad != 0;
}

static int case_constant_values(hipStream_t s) {
  const int B = 3, H = 2, N = 50, d = 32;
  const size_t n = (size_t)B * H * N * d;
  float* hq = malloc(n * 4); float* hk = malloc(n * 4);
  float* hv = malloc(n * 4); float* ho = malloc(n * 4);
  for (size_t i = 0; i < n; ++i) { hq[i] = next_val(); hk[i] = next_val(); }
  for (size_t i = 0; i < n; ++i) hv[i] = 0.25f * (float)((i % d) + 1) - 3.f;  /* row-independent */
  void *dq, *dk, *dv, *dout;
  HIP_OK(hipMalloc(&dq, n * 4)); HIP_OK(hipMalloc(&dk, n * 4));
  HIP_OK(hipMalloc(&dv, n * 4)); HIP_OK(hipMalloc(&dout, n * 4));
  HIP_OK(hipMemcpy(dq, hq, n * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, hk, n * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, hv, n * 4, hipMemcpyHostToDevice));
  attn_tensor_t q = tensor(dq, B, H, N, d), k = tensor(dk, B, H, N, d);
  attn_tensor_t v = tensor(dv, B, H, N, d), o = tensor(dout, B, H, N, d);
  int st = attn_fwd(&q, &k, &v, NULL, NULL, &o, ATTN_F32, s);
  if (st != ATTN_OK) { printf("FAIL constant values: attn_fwd %s\n", attn_strerror(st)); return 1; }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(ho, dout, n * 4, hipMemcpyDeviceToHost));
  double worst = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double e = fabs((double)ho[i] - (double)hv[i]);
    if (!(e <= worst)) worst = e;  /* also catches NaN */
  }
  const int bad = !(worst <= 1e-5);
  if (bad) printf("FAIL constant values: max abs err %.3e\n", worst);
  HIP_OK(hipFree(dq)); HIP_OK(hipFree(dk)); HIP_OK(hipFree(dv)); HIP_OK(hipFree(dout));
  free(hq); free(hk); free(hv); free(ho);
  return bad;
}

int main(void) {
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  printf("case: single key (bf16, 2x3x130, d=64)\n");
  fflush(stdout);
  int fails = case_single_key(s);
  printf("case: constant values (f32, 3x2x50, d=32)\n");
  fflush(stdout);
  fails += case_constant_values(s);
  HIP_OK(hipStreamDestroy(s));
  if (fails == 0) printf("ok\n");
  return fails == 0 ? 0 : 1;
}
