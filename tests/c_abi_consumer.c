/*
 * A plain C99 consumer of the library: it includes only include/bia.h, links
 * libbia.so and uses the host-side half of the ABI (planning, introspection,
 * status codes and messages), which needs no GPU. The expected work lists are
 * derived here from the split rule itself (keys [k * split, (k + 1) * split)
 * anchored at key 0; q tiles of 128 (token, head-in-group) rows, so 128 / g
 * tokens per tile), not taken from the library.
 *
 * Exit status 0 and a last line "ok" when every check holds.
 */
#include <stdio.h>
#include <string.h>

#include "bia.h"

static int failures = 0;

#define CHECK(cond, ...)                           \
  do {                                             \
    if (!(cond)) {                                 \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                \
      fputc('\n', stderr);                         \
      ++failures;                                  \
    }                                              \
  } while (0)

/* (q tile, partition) pairs of a causal prefill: request r's query token i
 * sits at position kv - qo + i and sees keys 0 .. that position. */
static int expected_prefill_items(const int32_t* qo, const int32_t* kv, int batch, int group,
                                  int split) {
  const int tile_tokens = 128 / group;
  int n = 0;
  for (int r = 0; r < batch; ++r) {
    const int q = qo[r + 1] - qo[r];
    const int k = kv[r + 1] - kv[r];
    for (int t0 = 0; t0 < q; t0 += tile_tokens) {
      const int last = t0 + tile_tokens < q ? t0 + tile_tokens - 1 : q - 1;
      const int last_pos = k - q + last;
      n += last_pos / split + 1;
    }
  }
  return n;
}

/* Real (non-padding) items of a plan and the sum of their query tokens. */
static void count_items(const bia_plan* plan, int* n_real, long* tokens, int* bad_begin,
                        int split) {
  static int32_t items[8 * 4096];
  const int n = bia_plan_num_items(plan);
  const int got = bia_plan_get_items(plan, items, n < 4096 ? n : 4096);
  *n_real = 0;
  *tokens = 0;
  *bad_begin = 0;
  for (int i = 0; i < got; ++i) {
    const int32_t* it = items + 8 * i;
    if (it[1] == 0) continue; /* n_tok 0: padding of the launch order */
    ++*n_real;
    *tokens += it[1];
    if (it[6] % split != 0) ++*bad_begin; /* kv_begin on the partition grid */
  }
}

int main(void) {
  /* two requests: 100 tokens from scratch, and a 172-token chunk over 128
   * cached tokens; GQA group 4 (32 tokens per q tile), D 64 */
  const int32_t qo[3] = {0, 100, 272};
  const int32_t kv[3] = {0, 100, 400};
  int32_t pages[7 + 19];
  for (int i = 0; i < 26; ++i) pages[i] = 63 - 2 * i;

  CHECK(bia_prefill_chunk_align() == 128, "chunk align %d", (int)bia_prefill_chunk_align());

  const int splits[2] = {4096, 64};
  for (int s = 0; s < 2; ++s) {
    bia_plan* plan = NULL;
    bia_status st = bia_plan_create(BIA_MODE_PREFILL, qo, kv, pages, 2, 4, 1, 64, 16, 64,
                                    splits[s], 0u, &plan);
    CHECK(st == BIA_OK && plan != NULL, "prefill plan split %d: %d %s", splits[s], (int)st,
          bia_last_error());
    if (plan == NULL) continue;
    int n_real, bad_begin;
    long tokens;
    count_items(plan, &n_real, &tokens, &bad_begin, splits[s]);
    const int want = expected_prefill_items(qo, kv, 2, 4, splits[s]);
    CHECK(n_real == want, "split %d: %d items, expected %d", splits[s], n_real, want);
    CHECK(bad_begin == 0, "split %d: %d items off the partition grid", splits[s], bad_begin);
    /* every query token appears once per partition its tile reaches; at one
     * partition per row (split 4096) that is exactly once */
    if (splits[s] == 4096) {
      CHECK(tokens == 272, "split 4096: %ld query tokens in items, expected 272", tokens);
      CHECK(bia_plan_num_states(plan) == 0, "split 4096: partial states %lld",
            (long long)bia_plan_num_states(plan));
    } else {
      CHECK(bia_plan_num_states(plan) > 0, "split 64: no partial states");
    }
    CHECK(bia_plan_workspace_bytes(plan) > 0, "split %d: empty workspace", splits[s]);
    bia_plan_destroy(plan);
  }

  /* decode: kv 1, 2048, 2049 at split 2048 -> 1 + 1 + 2 partitions per kv head */
  {
    const int32_t dq[4] = {0, 1, 2, 3};
    const int32_t dk[4] = {0, 1, 2049, 4098};
    static int32_t dpages[1 + 128 + 129];
    for (int i = 0; i < 258; ++i) dpages[i] = i;
    bia_plan* plan = NULL;
    bia_status st = bia_plan_create(BIA_MODE_DECODE, dq, dk, dpages, 3, 32, 8, 128, 16, 1024,
                                    2048, 0u, &plan);
    CHECK(st == BIA_OK && plan != NULL, "decode plan: %d %s", (int)st, bia_last_error());
    if (plan != NULL) {
      int n_real, bad_begin;
      long tokens;
      count_items(plan, &n_real, &tokens, &bad_begin, 2048);
      CHECK(n_real == 4 * 8, "decode: %d items, expected 32", n_real);
      CHECK(bad_begin == 0, "decode: %d items off the partition grid", bad_begin);
      CHECK(bia_plan_num_states(plan) > 0, "decode: the 2049-key request has no states");
      bia_plan_destroy(plan);
    }
  }

  /* status codes, each with a message, and no plan handed out */
  {
    bia_plan* plan = NULL;
    bia_status st = bia_plan_create(BIA_MODE_PREFILL, qo, kv, pages, 2, 4, 1, 64, 16, 64, 100,
                                    0u, &plan);
    CHECK(st == BIA_ERR_INVALID_ARG && plan == NULL, "split 100: %d", (int)st);
    CHECK(strlen(bia_last_error()) > 0, "split 100: no message");

    int32_t bad_pages[26];
    memcpy(bad_pages, pages, sizeof(bad_pages));
    bad_pages[25] = 64; /* == num_pages */
    st = bia_plan_create(BIA_MODE_PREFILL, qo, kv, bad_pages, 2, 4, 1, 64, 16, 64, 4096, 0u,
                         &plan);
    CHECK(st == BIA_ERR_PAGE_RANGE && plan == NULL, "page 64 of 64: %d", (int)st);

    const int32_t long_qo[3] = {0, 100, 301}; /* qo 201 > kv 200 */
    const int32_t short_kv[3] = {0, 100, 300};
    st = bia_plan_create(BIA_MODE_PREFILL, long_qo, short_kv, pages, 2, 4, 1, 64, 16, 64, 4096,
                         0u, &plan);
    CHECK(st == BIA_ERR_SHAPE && plan == NULL, "qo > kv: %d", (int)st);

    st = bia_plan_create(BIA_MODE_PREFILL, qo, kv, pages, 2, 4, 1, 96, 16, 64, 4096, 0u, &plan);
    CHECK(st == BIA_ERR_UNSUPPORTED && plan == NULL, "head_dim 96: %d", (int)st);

    st = bia_plan_create(BIA_MODE_DECODE, qo, kv, pages, 2, 4, 1, 64, 16, 64, 2048, 0u, &plan);
    CHECK(st != BIA_OK && plan == NULL, "decode with qo_len 100 accepted");

    /* the 172-token chunk starts at key 128: on the grid; one starting at
     * key 100 is not, and the strict flag rejects it */
    st = bia_plan_create(BIA_MODE_PREFILL, qo, kv, pages, 2, 4, 1, 64, 16, 64, 4096,
                         BIA_PLAN_STRICT_CHUNK_ALIGN, &plan);
    CHECK(st == BIA_OK, "strict, on-grid chunk: %d %s", (int)st, bia_last_error());
    bia_plan_destroy(plan);
    plan = NULL;
    const int32_t off_qo[3] = {0, 100, 300};  /* second request: qo 200 over kv 300 */
    st = bia_plan_create(BIA_MODE_PREFILL, off_qo, kv, pages, 2, 4, 1, 64, 16, 64, 4096,
                         BIA_PLAN_STRICT_CHUNK_ALIGN, &plan);
    CHECK(st == BIA_ERR_INVALID_ARG && plan == NULL, "strict, chunk at key 100: %d", (int)st);
    CHECK(strstr(bia_last_error(), "aligned to 128") != NULL, "strict message: %s",
          bia_last_error());
  }

  bia_plan_destroy(NULL); /* a no-op */

  if (failures != 0) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
