// Host split planner: validates a batch and lays out its work list.
//
// The layout is a function of each request's (qo_len, kv_len) alone: q tiles
// start at the request's first query token and hold 128 / group tokens (64 /
// group for latent plans);
// split-KV partitions are [k * split, (k + 1) * split) anchored at key 0 of
// the request (a fixed split size, sglang PR #10417, Modifications; the
// 128-row q-tile grid, sglang PR #43612, Summary). The launch order of the
// items (XCD-aware for prefill, longest first for decode) changes nothing in
// any result.
//
// Plain C++: no HIP call, so it runs and is tested without a GPU.
#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "plan.h"

namespace bia {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

bia_status fail(bia_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Keys of a work item: [kv_begin, min(kv_begin + split, last_pos + 1)).
static int64_t item_tiles(const WorkItem& w, int32_t split) {
  int64_t last = static_cast<int64_t>(w.pos0) + w.n_tok - 1;
  int64_t end = std::min<int64_t>(static_cast<int64_t>(w.kv_begin) + split, last + 1);
  return ceil_div(end - w.kv_begin, kKvTile);
}

// Prefill launch order. Workgroup i runs on XCD i mod 8, and each XCD has its
// own L2; the q tiles of one (request, kv head) pair all read the same K/V
// pages. So the items are grouped into units (a pair, or for batches with few
// pairs a round-robin share of a pair's items), units are spread over the 8
// XCDs by work (largest first, each to the least-loaded XCD), each XCD runs
// its units one after the other with every unit's items longest first, and
// the per-XCD lists are interleaved so that launch index 8 s + x is item s of
// XCD x (shorter lists padded with empty items). The XCD's running
// workgroups then share one pair's pages in its L2 instead of thrashing it
// with all pairs at once. The order changes no result.
constexpr int kXcds = 8;
constexpr size_t kMinUnits = 4 * kXcds;

static void order_for_xcds(PlanData& d, const std::vector<int64_t>& unit_of) {
  const int32_t split = d.split;
  const size_t n = d.items.size();
  if (n == 0) return;
  // units in order of first appearance
  std::vector<std::vector<size_t>> units;
  {
    std::vector<std::pair<int64_t, size_t>> key(n);
    for (size_t i = 0; i < n; ++i) key[i] = {unit_of[i], i};
    std::stable_sort(key.begin(), key.end(),
                     [](const auto& a, const auto& b) { return a.first < b.first; });
    for (size_t i = 0; i < n; ++i) {
      if (i == 0 || key[i].first != key[i - 1].first) units.emplace_back();
      units.back().push_back(key[i].second);
    }
  }
  auto longest_first = [&](std::vector<size_t>& v) {
    std::stable_sort(v.begin(), v.end(), [&](size_t a, size_t b) {
      return item_tiles(d.items[a], split) > item_tiles(d.items[b], split);
    });
  };
  for (auto& u : units) longest_first(u);
  if (units.size() < kMinUnits) {  // few pairs: deal each pair's items into k shares
    const size_t k = (kMinUnits + units.size() - 1) / units.size();
    std::vector<std::vector<size_t>> shares;
    for (const auto& u : units) {
      const size_t first = shares.size();
      shares.resize(first + std::min(k, u.size()));
      for (size_t i = 0; i < u.size(); ++i) shares[first + i % k].push_back(u[i]);
    }
    units.swap(shares);
  }
  std::vector<int64_t> work(units.size(), 0);
  for (size_t u = 0; u < units.size(); ++u)
    for (size_t i : units[u]) work[u] += item_tiles(d.items[i], split);
  std::vector<size_t> by_work(units.size());
  for (size_t u = 0; u < units.size(); ++u) by_work[u] = u;
  std::stable_sort(by_work.begin(), by_work.end(),
                   [&](size_t a, size_t b) { return work[a] > work[b]; });
  std::vector<std::vector<size_t>> xcd(kXcds);
  int64_t load[kXcds] = {0};
  for (size_t u : by_work) {
    int best = 0;
    for (int x = 1; x < kXcds; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += work[u];
    xcd[best].insert(xcd[best].end(), units[u].begin(), units[u].end());
  }
  size_t longest = 0;
  for (const auto& l : xcd) longest = std::max(longest, l.size());
  std::vector<WorkItem> out;
  out.reserve(longest * kXcds);
  const WorkItem empty{0, 0, 0, 0, 0, 0, 0, -1};
  for (size_t s = 0; s < longest; ++s)
    for (int x = 0; x < kXcds; ++x)
      out.push_back(s < xcd[x].size() ? d.items[xcd[x][s]] : empty);
  // trailing padding launches nothing useful: drop it
  while (!out.empty() && out.back().n_tok == 0) out.pop_back();
  d.items.swap(out);
}

static bia_status build(PlanData& d, const int32_t* qo_indptr,
                        const int32_t* kv_indptr) {
  const bool decode = d.mode == BIA_MODE_DECODE;
  const int32_t g = d.group;
  const int32_t T = decode ? 1 : d.tile_tokens;
  std::vector<int64_t> unit_of;  // (request, kv head) of each item
  int64_t page_off = 0;
  for (int32_t r = 0; r < d.batch; ++r) {
    const int32_t qo_len = qo_indptr[r + 1] - qo_indptr[r];
    const int32_t kv_len = kv_indptr[r + 1] - kv_indptr[r];
    for (int32_t t0 = 0; t0 < qo_len; t0 += kAppendTokens)
      d.appends.push_back(AppendItem{qo_indptr[r] + t0, std::min(kAppendTokens, qo_len - t0),
                                     kv_len - qo_len + t0, static_cast<int32_t>(page_off)});
    for (int32_t t0 = 0; t0 < qo_len; t0 += T) {
      const int32_t n_tok = std::min(T, qo_len - t0);
      const int32_t pos0 = kv_len - qo_len + t0;
      const int64_t last = static_cast<int64_t>(pos0) + n_tok - 1;
      const int32_t n_splits = static_cast<int32_t>(last / d.split + 1);
      const int32_t rows = n_tok * g;
      for (int32_t h = 0; h < d.num_kv_heads; ++h) {
        int64_t base = -1;
        if (n_splits > 1) {
          base = d.n_states;
          d.n_states += static_cast<int64_t>(n_splits) * rows;
          if (d.n_states > INT32_MAX)
            return fail(BIA_ERR_SHAPE, "plan needs %lld partial states (> 2^31)",
                        static_cast<long long>(d.n_states));
          d.merges.push_back(MergeItem{static_cast<int32_t>(base), n_splits,
                                       qo_indptr[r] + t0, n_tok, h, rows, 0, 0});
        }
        for (int32_t k = 0; k < n_splits; ++k) {
          WorkItem w{qo_indptr[r] + t0, n_tok, pos0, kv_len,
                     static_cast<int32_t>(page_off), h, k * d.split,
                     base < 0 ? -1 : static_cast<int32_t>(base + int64_t(k) * rows)};
          d.items.push_back(w);
          unit_of.push_back(static_cast<int64_t>(r) * d.num_kv_heads + h);
        }
      }
    }
    page_off += ceil_div(kv_len, d.page_size);
  }
  if (d.items.size() > static_cast<size_t>(INT32_MAX))
    return fail(BIA_ERR_SHAPE, "too many work items");
  if (!decode) {
    order_for_xcds(d, unit_of);
    if (d.items.size() > static_cast<size_t>(INT32_MAX))
      return fail(BIA_ERR_SHAPE, "too many work items");
    return BIA_OK;
  }
  // Decode items share no pages: longest first, so the tail of the launch is
  // short work. Whole partitions first, in (request, kv head, partition)
  // order, then the partial last partitions by 64-key tiles (a stable sort:
  // ties keep request, kv head order). The device planner of the
  // graph-capturable decode launches the same order.
  const int32_t split = d.split;
  auto whole = [split](const WorkItem& w) { return w.kv_len - w.kv_begin >= split; };
  std::stable_sort(d.items.begin(), d.items.end(),
                   [split, whole](const WorkItem& a, const WorkItem& b) {
                     if (whole(a) != whole(b)) return whole(a);
                     return item_tiles(a, split) > item_tiles(b, split);
                   });
  return BIA_OK;
}

}  // namespace bia

using namespace bia;

// Head counts, head dim, page size, pool size and split size every plan kind
// shares.
static bia_status check_shape(int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t num_pages, int32_t split_size) {
  if (num_qo_heads <= 0 || num_kv_heads <= 0)
    return fail(BIA_ERR_INVALID_ARG, "head counts must be positive (%d, %d)",
                num_qo_heads, num_kv_heads);
  if (num_qo_heads % num_kv_heads != 0)
    return fail(BIA_ERR_SHAPE, "num_qo_heads %d is not a multiple of num_kv_heads %d",
                num_qo_heads, num_kv_heads);
  const int32_t group = num_qo_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(BIA_ERR_UNSUPPORTED, "GQA group %d not supported (1, 2, 4, 8)", group);
  if (head_dim != 64 && head_dim != 128)
    return fail(BIA_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)", head_dim);
  if (page_size != kPageSize)
    return fail(BIA_ERR_UNSUPPORTED, "page_size %d not supported (16)", page_size);
  if (num_pages < 0) return fail(BIA_ERR_INVALID_ARG, "num_pages %d < 0", num_pages);
  if (split_size <= 0 || split_size % kKvTile != 0)
    return fail(BIA_ERR_INVALID_ARG,
                "split_size %d must be a positive multiple of the %d-key KV tile",
                split_size, kKvTile);
  return BIA_OK;
}

bia_status bia::plan_create_host(bia_mode mode, const int32_t* qo_indptr,
                                 const int32_t* kv_indptr, const int32_t* page_table,
                                 int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t page_size, int32_t num_pages,
                                 int32_t split_size, uint32_t flags, bia_plan** out_plan) {
  if (out_plan == nullptr) return fail(BIA_ERR_INVALID_ARG, "out_plan is NULL");
  *out_plan = nullptr;
  if (mode != BIA_MODE_PREFILL && mode != BIA_MODE_DECODE)
    return fail(BIA_ERR_INVALID_ARG, "unknown mode %d", static_cast<int>(mode));
  if (batch < 0) return fail(BIA_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (batch > 0 && (qo_indptr == nullptr || kv_indptr == nullptr))
    return fail(BIA_ERR_INVALID_ARG, "qo_indptr / kv_indptr is NULL");
  if ((flags & ~(BIA_PLAN_STRICT_CHUNK_ALIGN | BIA_PLAN_MLA)) != 0)
    return fail(BIA_ERR_INVALID_ARG, "unknown plan flags 0x%x", flags);
  const bool mla = (flags & BIA_PLAN_MLA) != 0;
  int32_t group = 0;
  if (mla) {
    if (num_kv_heads != 1)
      return fail(BIA_ERR_SHAPE, "an MLA plan has one cached head, got num_kv_heads %d",
                  num_kv_heads);
    if (head_dim != BIA_MLA_QK_DIM)
      return fail(BIA_ERR_UNSUPPORTED, "MLA head_dim %d not supported (%d)", head_dim,
                  BIA_MLA_QK_DIM);
    if (num_qo_heads != 8 && num_qo_heads != 16 && num_qo_heads != 32 && num_qo_heads != 64 &&
        num_qo_heads != 128)
      return fail(BIA_ERR_UNSUPPORTED, "MLA num_qo_heads %d not supported (8 .. 128, a power "
                  "of 2)", num_qo_heads);
    if (page_size != kPageSize)
      return fail(BIA_ERR_UNSUPPORTED, "page_size %d not supported (16)", page_size);
    if (num_pages < 0) return fail(BIA_ERR_INVALID_ARG, "num_pages %d < 0", num_pages);
    if (split_size <= 0 || split_size % kKvTile != 0)
      return fail(BIA_ERR_INVALID_ARG,
                  "split_size %d must be a positive multiple of the %d-key KV tile",
                  split_size, kKvTile);
    if (split_size > BIA_MLA_MAX_SPLIT)
      return fail(BIA_ERR_UNSUPPORTED, "MLA split_size %d above %d", split_size,
                  BIA_MLA_MAX_SPLIT);
    group = std::min(num_qo_heads, kMlaTileRows);  // q heads per head block
  } else {
    const bia_status shape_st =
        check_shape(num_qo_heads, num_kv_heads, head_dim, page_size, num_pages, split_size);
    if (shape_st != BIA_OK) return shape_st;
    group = num_qo_heads / num_kv_heads;
  }
  int64_t total_pages = 0;
  if (batch > 0) {
    if (qo_indptr[0] != 0 || kv_indptr[0] != 0)
      return fail(BIA_ERR_SHAPE, "indptr arrays must start at 0");
    for (int32_t r = 0; r < batch; ++r) {
      const int64_t qo = int64_t(qo_indptr[r + 1]) - qo_indptr[r];
      const int64_t kv = int64_t(kv_indptr[r + 1]) - kv_indptr[r];
      if (qo < 0 || kv < 0)
        return fail(BIA_ERR_SHAPE, "request %d: indptr decreases", r);
      if (qo > kv)
        return fail(BIA_ERR_SHAPE, "request %d: qo_len %lld > kv_len %lld", r,
                    static_cast<long long>(qo), static_cast<long long>(kv));
      if (mode == BIA_MODE_DECODE && qo != 1)
        return fail(BIA_ERR_SHAPE, "request %d: decode needs qo_len 1, got %lld", r,
                    static_cast<long long>(qo));
      if (mode == BIA_MODE_PREFILL && (flags & BIA_PLAN_STRICT_CHUNK_ALIGN) && qo > 0 &&
          (kv - qo) % kQTileRows != 0)
        return fail(BIA_ERR_INVALID_ARG,
                    "request %d: chunk starts at token %lld, not aligned to %d tokens", r,
                    static_cast<long long>(kv - qo), kQTileRows);
      total_pages += ceil_div(kv, page_size);
    }
    if (total_pages > 0 && page_table == nullptr)
      return fail(BIA_ERR_INVALID_ARG, "page_table is NULL");
    for (int64_t i = 0; i < total_pages; ++i) {
      if (page_table[i] < 0 || page_table[i] >= num_pages)
        return fail(BIA_ERR_PAGE_RANGE, "page_table[%lld] = %d outside [0, %d)",
                    static_cast<long long>(i), page_table[i], num_pages);
    }
    if (total_pages > INT32_MAX)
      return fail(BIA_ERR_SHAPE, "page table longer than 2^31 entries");
  }

  bia_plan* plan = new (std::nothrow) bia_plan();
  if (plan == nullptr) return fail(BIA_ERR_INVALID_ARG, "out of host memory");
  PlanData& d = plan->d;
  d.mode = mode;
  d.batch = batch;
  d.num_qo_heads = num_qo_heads;
  d.num_kv_heads = mla ? num_qo_heads / group : num_kv_heads;
  d.head_dim = head_dim;
  d.mla = mla;
  d.v_dim = mla ? BIA_MLA_V_DIM : head_dim;
  d.page_size = page_size;
  d.num_pages = num_pages;
  d.split = split_size;
  d.flags = flags;
  d.group = group;
  d.tile_tokens = (mla ? kMlaTileRows : kQTileRows) / group;
  d.total_q = batch > 0 ? qo_indptr[batch] : 0;
  d.n_states = 0;
  bia_status st = BIA_OK;
  try {
    st = build(d, qo_indptr, kv_indptr);
  } catch (const std::bad_alloc&) {
    st = fail(BIA_ERR_INVALID_ARG, "out of host memory while planning");
  }
  if (st != BIA_OK) {
    delete plan;
    return st;
  }
  d.off_items = 0;
  d.off_merges = d.items.size() * sizeof(WorkItem);
  d.off_appends = d.off_merges + d.merges.size() * sizeof(MergeItem);
  d.blob_bytes = d.off_appends + d.appends.size() * sizeof(AppendItem);
  d.off_o = align_up(d.blob_bytes, kWsAlign);
  d.off_lse = align_up(d.off_o + size_t(d.n_states) * d.v_dim * sizeof(float), kWsAlign);
  d.ws_bytes = d.n_states > 0 ? d.off_lse + size_t(d.n_states) * sizeof(float)
                              : align_up(d.blob_bytes, kWsAlign);
  d.blob.resize(d.blob_bytes);
  if (!d.items.empty())
    std::memcpy(d.blob.data() + d.off_items, d.items.data(),
                d.items.size() * sizeof(WorkItem));
  if (!d.merges.empty())
    std::memcpy(d.blob.data() + d.off_merges, d.merges.data(),
                d.merges.size() * sizeof(MergeItem));
  if (!d.appends.empty())
    std::memcpy(d.blob.data() + d.off_appends, d.appends.data(),
                d.appends.size() * sizeof(AppendItem));
  *out_plan = plan;
  return BIA_OK;
}

void bia::plan_free_host(bia_plan* plan) { delete plan; }

extern "C" size_t bia_plan_workspace_bytes(const bia_plan* plan) {
  return plan == nullptr ? 0 : plan->d.ws_bytes;
}

extern "C" int32_t bia_plan_num_items(const bia_plan* plan) {
  return plan == nullptr ? 0 : static_cast<int32_t>(plan->d.items.size());
}

extern "C" int32_t bia_plan_get_items(const bia_plan* plan, int32_t* items, int32_t n) {
  if (plan == nullptr || items == nullptr || n <= 0) return 0;
  const int32_t m = std::min<int32_t>(n, static_cast<int32_t>(plan->d.items.size()));
  std::memcpy(items, plan->d.items.data(), size_t(m) * sizeof(WorkItem));
  return m;
}

extern "C" int64_t bia_plan_num_states(const bia_plan* plan) {
  return plan == nullptr ? 0 : plan->d.n_states;
}

extern "C" bia_status bia_decode_graph_create(int32_t max_batch, int32_t num_qo_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t page_size, int32_t num_pages,
                                              int32_t max_kv_len, int32_t page_table_capacity,
                                              int32_t split_size, bia_decode_graph** out) {
  if (out == nullptr) return fail(BIA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const bia_status shape_st =
      check_shape(num_qo_heads, num_kv_heads, head_dim, page_size, num_pages, split_size);
  if (shape_st != BIA_OK) return shape_st;
  if (max_batch <= 0) return fail(BIA_ERR_INVALID_ARG, "max_batch %d must be positive", max_batch);
  if (max_kv_len <= 0)
    return fail(BIA_ERR_INVALID_ARG, "max_kv_len %d must be positive", max_kv_len);
  if (page_table_capacity < 0)
    return fail(BIA_ERR_INVALID_ARG, "page_table_capacity %d < 0", page_table_capacity);
  const int32_t group = num_qo_heads / num_kv_heads;
  const int64_t max_splits = ceil_div(max_kv_len, split_size);
  const int64_t n_items = int64_t(max_batch) * num_kv_heads * max_splits;
  const int64_t n_states = n_items * group;
  if (n_items > INT32_MAX || n_states > INT32_MAX)
    return fail(BIA_ERR_SHAPE, "capacity needs %lld partial states (> 2^31)",
                static_cast<long long>(n_states));
  bia_decode_graph* dg = new (std::nothrow) bia_decode_graph();
  if (dg == nullptr) return fail(BIA_ERR_INVALID_ARG, "out of host memory");
  DecodeGraphData& d = dg->d;
  d.max_batch = max_batch;
  d.num_qo_heads = num_qo_heads;
  d.num_kv_heads = num_kv_heads;
  d.head_dim = head_dim;
  d.page_size = page_size;
  d.num_pages = num_pages;
  d.max_kv_len = max_kv_len;
  d.page_table_capacity = page_table_capacity;
  d.split = split_size;
  d.group = group;
  d.max_splits = static_cast<int32_t>(max_splits);
  d.n_items = n_items;
  d.n_merges = int64_t(max_batch) * num_kv_heads;
  d.n_states = n_states;
  d.off_flags = 0;
  d.off_items = align_up(size_t(max_batch) * sizeof(int32_t), kWsAlign);
  d.off_merges = align_up(d.off_items + size_t(n_items) * sizeof(WorkItem), kWsAlign);
  d.off_o = align_up(d.off_merges + size_t(d.n_merges) * sizeof(MergeItem), kWsAlign);
  d.off_lse = align_up(d.off_o + size_t(n_states) * head_dim * sizeof(float), kWsAlign);
  d.ws_bytes = align_up(d.off_lse + size_t(n_states) * sizeof(float), kWsAlign);
  *out = dg;
  return BIA_OK;
}

extern "C" size_t bia_decode_graph_workspace_bytes(const bia_decode_graph* dg) {
  return dg == nullptr ? 0 : dg->d.ws_bytes;
}

extern "C" void bia_decode_graph_destroy(bia_decode_graph* dg) { delete dg; }

extern "C" int32_t bia_prefill_chunk_align(void) { return kQTileRows; }

extern "C" const char* bia_last_error(void) { return g_last_error.c_str(); }
