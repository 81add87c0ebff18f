/*
 * A plain C99 program that runs a paged decode on the GPU through include/bia.h
 * alone: device memory from the HIP runtime API, no Python, no torch. The
 * inputs are chosen so the result has a closed form: every key of a kv head
 * is the same vector, so each request's scores are all equal, its softmax
 * weights are uniform, and its output is the mean of the values it sees, with
 * lse = (the common scaled logit) + ln(kv_len). One request of 5000 keys spans
 * three 2048-key partitions, so the fixed-order merge is exercised too.
 *
 * Exit status 0 and a last line "ok" when the outputs meet the closed form
 * within 2e-2 (out) and 1e-3 (lse).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bia.h"

enum { B = 3, HQ = 32, HKV = 8, G = HQ / HKV, D = 128, PAGE = 16, NUM_PAGES = 1024 };
static const int32_t kKvLen[B] = {1, 777, 5000};

/* bf16 from a float that is exactly representable in bf16 (all values here
 * are multiples of 1/64 within [-1, 1]) */
static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static double double_of_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}
static double key_val(int h, int d) { return (double)(((h * 37 + d * 11) % 33) - 16) / 64.0; }
static double value_val(int j, int h, int d) {
  return (double)(((j * 131 + h * 17 + d * 7) % 61) - 30) / 64.0;
}
static double query_val(int r, int hq, int d) {
  return (double)(((r * 29 + hq * 13 + d * 5) % 41) - 20) / 64.0;
}

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
      return 1;                                                             \
    }                                                                       \
  } while (0)

int main(void) {
  int32_t qo[B + 1], kv[B + 1];
  qo[0] = kv[0] = 0;
  int n_pages = 0;
  for (int r = 0; r < B; ++r) {
    qo[r + 1] = qo[r] + 1;
    kv[r + 1] = kv[r] + kKvLen[r];
    n_pages += (kKvLen[r] + PAGE - 1) / PAGE;
  }
  /* pages of all requests, scattered over the pool (a fixed odd stride) */
  int32_t* pages = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_pages);
  for (int i = 0; i < n_pages; ++i) pages[i] = (int32_t)((i * 389L + 5) % NUM_PAGES);

  const size_t pool_elems = (size_t)NUM_PAGES * PAGE * HKV * D;
  uint16_t* k_host = (uint16_t*)calloc(pool_elems, 2);
  uint16_t* v_host = (uint16_t*)calloc(pool_elems, 2);
  uint16_t* q_host = (uint16_t*)malloc((size_t)B * HQ * D * 2);
  int page_off = 0;
  for (int r = 0; r < B; ++r) {
    for (int j = 0; j < kKvLen[r]; ++j) {
      const size_t row = ((size_t)pages[page_off + j / PAGE] * PAGE + (size_t)(j % PAGE)) * HKV;
      for (int h = 0; h < HKV; ++h)
        for (int d = 0; d < D; ++d) {
          k_host[(row + (size_t)h) * D + (size_t)d] = bf16_of((float)key_val(h, d));
          v_host[(row + (size_t)h) * D + (size_t)d] = bf16_of((float)value_val(j, h, d));
        }
    }
    page_off += (kKvLen[r] + PAGE - 1) / PAGE;
    for (int hq = 0; hq < HQ; ++hq)
      for (int d = 0; d < D; ++d)
        q_host[((size_t)r * HQ + (size_t)hq) * D + (size_t)d] = bf16_of((float)query_val(r, hq, d));
  }

  const float sm_scale = 0.08838834764831845f; /* 1 / sqrt(128) */
  bia_plan* plan = NULL;
  bia_status st = bia_plan_create(BIA_MODE_DECODE, qo, kv, pages, B, HQ, HKV, D, PAGE,
                                  NUM_PAGES, BIA_DECODE_SPLIT, 0u, &plan);
  if (st != BIA_OK) {
    fprintf(stderr, "bia_plan_create: %d %s\n", (int)st, bia_last_error());
    return 1;
  }
  const size_t ws_bytes = bia_plan_workspace_bytes(plan);

  void *q_d, *k_d, *v_d, *out_d, *ws_d;
  int32_t* pt_d;
  float* lse_d;
  HIP_OK(hipMalloc(&q_d, (size_t)B * HQ * D * 2));
  HIP_OK(hipMalloc(&k_d, pool_elems * 2));
  HIP_OK(hipMalloc(&v_d, pool_elems * 2));
  HIP_OK(hipMalloc((void**)&pt_d, sizeof(int32_t) * (size_t)n_pages));
  HIP_OK(hipMalloc(&out_d, (size_t)B * HQ * D * 2));
  HIP_OK(hipMalloc((void**)&lse_d, sizeof(float) * B * HQ));
  HIP_OK(hipMalloc(&ws_d, ws_bytes > 256 ? ws_bytes : 256));
  HIP_OK(hipMemcpy(q_d, q_host, (size_t)B * HQ * D * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k_d, k_host, pool_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v_d, v_host, pool_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(pt_d, pages, sizeof(int32_t) * (size_t)n_pages, hipMemcpyHostToDevice));

  st = bia_decode_paged(plan, q_d, k_d, v_d, pt_d, sm_scale, out_d, lse_d, ws_d, ws_bytes,
                        NULL);
  if (st != BIA_OK) {
    fprintf(stderr, "bia_decode_paged: %d %s\n", (int)st, bia_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  uint16_t* out_host = (uint16_t*)malloc((size_t)B * HQ * D * 2);
  float lse_host[B * HQ];
  HIP_OK(hipMemcpy(out_host, out_d, (size_t)B * HQ * D * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse_host, lse_d, sizeof(lse_host), hipMemcpyDeviceToHost));

  double err_out = 0.0, err_lse = 0.0;
  for (int r = 0; r < B; ++r)
    for (int hq = 0; hq < HQ; ++hq) {
      const int h = hq / G;
      double logit = 0.0;
      for (int d = 0; d < D; ++d) logit += query_val(r, hq, d) * key_val(h, d);
      const double lse_ref = (double)sm_scale * logit + log((double)kKvLen[r]);
      const double e = fabs((double)lse_host[r * HQ + hq] - lse_ref);
      if (!(e <= err_lse)) err_lse = e; /* NaN propagates as a failure */
      for (int d = 0; d < D; ++d) {
        double mean = 0.0;
        for (int j = 0; j < kKvLen[r]; ++j) mean += value_val(j, h, d);
        mean /= (double)kKvLen[r];
        const double got = double_of_bf16(out_host[((size_t)r * HQ + (size_t)hq) * D + (size_t)d]);
        const double eo = fabs(got - mean);
        if (!(eo <= err_out)) err_out = eo;
      }
    }
  printf("max |out - mean of V| = %.3e, max |lse - closed form| = %.3e\n", err_out, err_lse);

  bia_plan_destroy(plan);
  hipFree(q_d);
  hipFree(k_d);
  hipFree(v_d);
  hipFree(pt_d);
  hipFree(out_d);
  hipFree(lse_d);
  hipFree(ws_d);
  free(pages);
  free(k_host);
  free(v_host);
  free(q_host);
  free(out_host);
  if (!(err_out <= 2e-2) || !(err_lse <= 1e-3)) {
    fprintf(stderr, "closed form not met\n");
    return 1;
  }
  printf("ok\n");
  return 0;
}
