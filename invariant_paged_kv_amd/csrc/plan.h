// Internal plan structures shared by the host planner (plan.cpp, plain C++)
// and the launch layer (bia.hip).
#ifndef BIA_PLAN_INTERNAL_H_
#define BIA_PLAN_INTERNAL_H_

#include <cstddef>
#include <cstdint>
#include <vector>

#include "bia.h"

namespace bia {

// One workgroup's work: one q tile of one kv head of one request, over one
// split-KV partition. For decode a "tile" is the single query token.
//   q_row0   global index (into q / out) of the tile's first query token
//   n_tok    query tokens in the tile (<= 128 / group; ragged last tile)
//   pos0     absolute KV position of the tile's first token
//   kv_len   the request's key count
//   page_off index in the page table of the request's first page
//   kv_head  kv head (its q heads are kv_head * group .. + group - 1)
//   kv_begin first key of the partition (a multiple of the split size)
//   state    -1: the tile's rows have one partition, write out/lse directly;
//            >= 0: first partial-state slot of this (tile, partition); row x
//            of the tile (x = token * group + head-in-group) uses slot
//            state + x.
struct WorkItem {
  int32_t q_row0, n_tok, pos0, kv_len, page_off, kv_head, kv_begin, state;
};

// Fixed-order merge of a tile whose rows span several partitions: row x
// folds slots state0 + k * stride + x for k = 0 .. n_splits - 1, ascending.
struct MergeItem {
  int32_t state0, n_splits, q_row0, n_tok, kv_head, stride, pad0, pad1;
};

// Copy of up to kAppendTokens new tokens of one request into its pages:
// rows src_row0 .. src_row0 + n_tok - 1 of k_new / v_new go to KV positions
// dst_pos0 .. ; the request's pages start at page_table[page_off].
struct AppendItem {
  int32_t src_row0, n_tok, dst_pos0, page_off;
};
constexpr int kAppendTokens = 16;

static_assert(sizeof(WorkItem) == 32, "work item is 8 int32");
static_assert(sizeof(AppendItem) == 16, "append item is 4 int32");
static_assert(sizeof(MergeItem) == 32, "merge item is 8 int32");

constexpr int kQTileRows = BIA_Q_TILE_ROWS;
constexpr int kMlaTileRows = 128;  // q rows of one latent-attention work item
constexpr int kKvTile = BIA_KV_TILE;
constexpr int kPageSize = BIA_PAGE_SIZE;
constexpr size_t kWsAlign = 256;

struct PlanData {
  bia_mode mode;
  int32_t batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_pages;
  int32_t split, group, tile_tokens;
  uint32_t flags;
  // Latent (MLA) plans: num_kv_heads counts head blocks of `group` q heads
  // (all reading the one cached head), head_dim is the q.k width (576) and
  // v_dim the output width (512); otherwise v_dim == head_dim.
  bool mla;
  int32_t v_dim;
  int64_t total_q;   // sum of qo_len: rows of q / out
  int64_t n_states;  // partial states written before the merge
  std::vector<WorkItem> items;
  std::vector<MergeItem> merges;
  std::vector<AppendItem> appends;
  // Workspace layout (byte offsets): [items | merges | appends] (the
  // uploaded blob), then fp32 o[n_states][head_dim], then fp32
  // lse[n_states].
  size_t off_items, off_merges, off_appends, off_o, off_lse, blob_bytes, ws_bytes;
  std::vector<unsigned char> blob;  // host copy of [items | merges | appends]
};

void set_error(const char* fmt, ...);
bia_status fail(bia_status st, const char* fmt, ...);

// The host half of bia_plan_create: validates the batch and builds the plan
// (work list, merge list, append list, workspace layout). Plain C++; the C
// entry point in the launch layer adds the pinned copy of the work list.
bia_status plan_create_host(bia_mode mode, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* page_table, int32_t batch, int32_t num_qo_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            int32_t num_pages, int32_t split_size, uint32_t flags,
                            bia_plan** out_plan);
// Frees the host part of a plan (the launch layer returns its pinned block
// first).
void plan_free_host(bia_plan* plan);

struct PinBlock;  // pinned work-list block of the launch layer's pool

// Fixed-capacity decode planned on the device (graph-capturable). Request r
// of a call has kv head h's partition s at item (r * Hkv + h) * max_splits + s
// and its merge at r * Hkv + h; partition s of (r, h) keeps its partial states
// at slots ((r * Hkv + h) * max_splits + s) * group + head-in-group.
struct DecodeGraphData {
  int32_t max_batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_pages;
  int32_t max_kv_len, page_table_capacity, split, group, max_splits;
  // Workspace layout (byte offsets): int32 flags[max_batch] | items | merges |
  // fp32 o[n_states][head_dim] | fp32 lse[n_states].
  int64_t n_items, n_merges, n_states;
  size_t off_flags, off_items, off_merges, off_o, off_lse, ws_bytes;
};

}  // namespace bia

// The opaque handles of the C ABI.
struct bia_plan {
  bia::PlanData d;
  // Pinned copy of d.blob, drawn from the launch layer's pool when the plan
  // is made (NULL when no GPU was visible then, or the blob is empty).
  bia::PinBlock* pin = nullptr;
};

struct bia_decode_graph {
  bia::DecodeGraphData d;
};

#endif  // BIA_PLAN_INTERNAL_H_
