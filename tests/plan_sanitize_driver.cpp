// Host planner under AddressSanitizer and UndefinedBehaviorSanitizer: builds
// with g++ from csrc/plan.cpp alone (no HIP) and drives the planner through
// valid and invalid batches, the introspection calls and the fixed-capacity
// decode handle. Exit status 0 when every call returned the expected status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "plan.h"

namespace {

int g_failures = 0;
int g_cases = 0;

struct Batch {
  std::vector<int32_t> qo, kv, pt;
};

Batch make(const std::vector<int32_t>& qo_lens, const std::vector<int32_t>& kv_lens,
           int32_t num_pages) {
  Batch b;
  b.qo.push_back(0);
  b.kv.push_back(0);
  int64_t pages = 0;
  for (size_t i = 0; i < qo_lens.size(); ++i) {
    b.qo.push_back(b.qo.back() + qo_lens[i]);
    b.kv.push_back(b.kv.back() + kv_lens[i]);
    pages += (kv_lens[i] + 15) / 16;
  }
  for (int64_t i = 0; i < pages; ++i)
    b.pt.push_back(static_cast<int32_t>((i * 7919) % (num_pages > 0 ? num_pages : 1)));
  return b;
}

// Plans the batch, checks the status, and reads everything back.
void run(const char* what, bia_mode mode, const Batch& b, int32_t hq, int32_t hkv, int32_t d,
         int32_t num_pages, int32_t split, uint32_t flags, bia_status want) {
  ++g_cases;
  bia_plan* plan = nullptr;
  const int32_t batch = static_cast<int32_t>(b.qo.size()) - 1;
  const bia_status st = bia::plan_create_host(
      mode, b.qo.data(), b.kv.data(), b.pt.empty() ? nullptr : b.pt.data(), batch, hq, hkv, d,
      16, num_pages, split, flags, &plan);
  if (st != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, st, want,
                 bia_last_error());
    ++g_failures;
  }
  if (st != BIA_OK) {
    if (plan != nullptr) {
      std::fprintf(stderr, "%s: failed plan was returned\n", what);
      ++g_failures;
    }
    if (std::strlen(bia_last_error()) == 0) {
      std::fprintf(stderr, "%s: no error message\n", what);
      ++g_failures;
    }
    return;
  }
  const int32_t n = bia_plan_num_items(plan);
  std::vector<int32_t> items(static_cast<size_t>(n) * 8 + 8, -7);
  const int32_t got = bia_plan_get_items(plan, items.data(), n);
  if (got != n || items[static_cast<size_t>(n) * 8] != -7) {
    std::fprintf(stderr, "%s: get_items wrote %d of %d or past the end\n", what, got, n);
    ++g_failures;
  }
  (void)bia_plan_get_items(plan, items.data(), n > 3 ? 3 : n);  // a short copy
  (void)bia_plan_num_states(plan);
  (void)bia_plan_workspace_bytes(plan);
  bia::plan_free_host(plan);
}

uint64_t g_lcg = 88172645463325252ull;
int32_t rnd(int32_t lo, int32_t hi) {  // [lo, hi]
  g_lcg = g_lcg * 6364136223846793005ull + 1442695040888963407ull;
  return lo + static_cast<int32_t>((g_lcg >> 33) % static_cast<uint64_t>(hi - lo + 1));
}

}  // namespace

int main() {
  const bia_mode P = BIA_MODE_PREFILL, DEC = BIA_MODE_DECODE;
  // validation paths (the same cases the Python ABI tests use)
  run("ok tiny", P, make({100, 300}, {100, 300}, 64), 4, 1, 64, 64, 4096, 0, BIA_OK);
  {
    Batch b = make({5, 0}, {10, 20}, 64);
    b.qo = {0, 5, 3};
    run("qo decreases", P, b, 4, 1, 64, 64, 4096, 0, BIA_ERR_SHAPE);
  }
  {
    Batch b = make({4}, {10}, 64);
    b.qo = {1, 5};
    run("indptr not at 0", P, b, 4, 1, 64, 64, 4096, 0, BIA_ERR_SHAPE);
  }
  run("qo > kv", P, make({11}, {10}, 64), 4, 1, 64, 64, 4096, 0, BIA_ERR_SHAPE);
  {
    Batch b = make({1}, {10}, 64);
    b.pt = {64};
    run("page id = num_pages", P, b, 4, 1, 64, 64, 4096, 0, BIA_ERR_PAGE_RANGE);
    b.pt = {-1};
    run("page id < 0", P, b, 4, 1, 64, 64, 4096, 0, BIA_ERR_PAGE_RANGE);
  }
  run("split 100", P, make({100}, {100}, 64), 4, 1, 64, 64, 100, 0, BIA_ERR_INVALID_ARG);
  run("split 0", P, make({100}, {100}, 64), 4, 1, 64, 64, 0, 0, BIA_ERR_INVALID_ARG);
  run("head_dim 96", P, make({100}, {100}, 64), 4, 1, 96, 64, 4096, 0, BIA_ERR_UNSUPPORTED);
  run("6 / 4 heads", P, make({100}, {100}, 64), 6, 4, 64, 64, 4096, 0, BIA_ERR_SHAPE);
  run("group 16", P, make({100}, {100}, 64), 48, 3, 64, 64, 4096, 0, BIA_ERR_UNSUPPORTED);
  run("decode qo 100", DEC, make({100}, {100}, 64), 4, 1, 64, 64, 4096, 0, BIA_ERR_SHAPE);
  run("mode 7", static_cast<bia_mode>(7), make({1}, {1}, 64), 4, 1, 64, 64, 4096, 0,
      BIA_ERR_INVALID_ARG);
  run("flag 4", P, make({1}, {1}, 64), 4, 1, 64, 64, 4096, 0x4, BIA_ERR_INVALID_ARG);
  run("strict ok", P, make({172}, {300}, 64), 4, 1, 64, 64, 4096, BIA_PLAN_STRICT_CHUNK_ALIGN,
      BIA_OK);
  run("strict off grid", P, make({200}, {300}, 64), 4, 1, 64, 64, 4096,
      BIA_PLAN_STRICT_CHUNK_ALIGN, BIA_ERR_INVALID_ARG);
  run("empty batch", P, make({}, {}, 0), 32, 8, 128, 0, 4096, 0, BIA_OK);
  run("MLA 8 kv heads", P, make({10}, {10}, 64), 16, 8, 576, 64, 4096, BIA_PLAN_MLA,
      BIA_ERR_SHAPE);
  run("MLA ok", P, make({10, 200}, {10, 900}, 128), 128, 1, 576, 128, 4096, BIA_PLAN_MLA,
      BIA_OK);
  run("MLA split too large", P, make({10}, {10}, 64), 16, 1, 576, 64, 32768, BIA_PLAN_MLA,
      BIA_ERR_UNSUPPORTED);
  {
    ++g_cases;
    bia_plan* plan = nullptr;
    if (bia::plan_create_host(P, nullptr, nullptr, nullptr, 2, 4, 1, 64, 16, 64, 4096, 0,
                              &plan) != BIA_ERR_INVALID_ARG ||
        bia::plan_create_host(P, nullptr, nullptr, nullptr, 0, 4, 1, 64, 16, 64, 4096, 0,
                              nullptr) != BIA_ERR_INVALID_ARG) {
      std::fprintf(stderr, "null arguments not rejected\n");
      ++g_failures;
    }
  }
  // seeded random batches: ragged prefill chunks, decode, every split, GQA
  // group and head dim
  const int32_t groups[4][2] = {{8, 8}, {16, 8}, {32, 8}, {64, 8}};
  for (int trial = 0; trial < 200; ++trial) {
    const int32_t batch = rnd(1, 64);
    const bool decode = trial % 3 == 2;
    std::vector<int32_t> qo, kv;
    for (int32_t r = 0; r < batch; ++r) {
      const int32_t k = rnd(decode ? 1 : 0, trial % 7 == 0 ? 70000 : 5000);
      kv.push_back(k);
      qo.push_back(decode ? 1 : rnd(0, k));
    }
    const int32_t pool = rnd(1, 1 << 17);
    // long contexts with a small split need more than 2^31 partial states
    // (a BIA_ERR_SHAPE case of its own, below): keep these splits >= 1024
    const int32_t split = trial % 7 == 0 ? 1024 * rnd(1, 8) : 64 * rnd(1, 80);
    const auto& g = groups[trial % 4];
    const int32_t d = trial % 2 ? 128 : 64;
    char what[64];
    std::snprintf(what, sizeof(what), "random trial %d", trial);
    run(what, decode ? DEC : P, make(qo, kv, pool), g[0], g[1], d, pool, split, 0, BIA_OK);
  }
  {
    // 64 requests of 70000 tokens at split 64: more than 2^31 partial states
    std::vector<int32_t> qo(64, 70000), kv(64, 70000);
    run("too many partial states", P, make(qo, kv, 1 << 17), 32, 8, 128, 1 << 17, 64, 0,
        BIA_ERR_SHAPE);
  }
  // fixed-capacity decode handles
  {
    ++g_cases;
    bia_decode_graph* dg = nullptr;
    if (bia_decode_graph_create(64, 32, 8, 128, 16, 131072, 32768, 131072, 2048, &dg) !=
            BIA_OK ||
        bia_decode_graph_workspace_bytes(dg) == 0) {
      std::fprintf(stderr, "decode graph create failed: %s\n", bia_last_error());
      ++g_failures;
    }
    bia_decode_graph_destroy(dg);
    bia_decode_graph* bad = nullptr;
    if (bia_decode_graph_create(0, 32, 8, 128, 16, 131072, 32768, 131072, 2048, &bad) ==
            BIA_OK ||
        bad != nullptr) {
      std::fprintf(stderr, "decode graph with max_batch 0 accepted\n");
      ++g_failures;
    }
    bia_decode_graph_destroy(nullptr);
  }
  if (bia_prefill_chunk_align() != 128) ++g_failures;
  std::printf("%d planner cases, %d failures\n", g_cases, g_failures);
  return g_failures == 0 ? 0 : 1;
}
