/*
 * bia.h — batch- and chunk-invariant attention over a paged KV cache, for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes is causal softmax attention of bf16 queries over
 * bf16 keys and values stored in fixed-size pages, split along the KV axis
 * into partitions of a fixed size, with the partial (o, lse) states of the
 * partitions merged in ascending partition order (sglang PR #10417 "[POC]
 * Support deterministic inference", Modifications: batch-invariant prefill
 * and decode, the paged prefill wrapper for every extend, a fixed split-KV of
 * 2048 tokens for decode and 4096 for prefill). Because the partition, the
 * merge order and every tile shape depend only on a request's own lengths,
 * a request's output bits do not depend on the batch it shares, on where its
 * pages sit in the pool, or on the GPU's compute-unit count; and a chunked
 * prefill whose chunks start on the 128-row q-tile grid reproduces the
 * unchunked prefill bit for bit (sglang PR #43612, commit message and
 * Summary: the fa2 q tile is 128 rows, 128 / gqa_group tokens).
 *
 * Conventions shared by every call:
 *   - B requests. qo_len_r = qo_indptr[r+1] - qo_indptr[r] new query tokens
 *     attend to kv_len_r = kv_indptr[r+1] - kv_indptr[r] keys, which already
 *     include this call's own tokens. Query i of request r sits at absolute
 *     position kv_len_r - qo_len_r + i and sees keys 0 .. that position
 *     (bottom-right causal alignment, so a chunk attends to its cached prefix).
 *   - Pages: P = 16 tokens. Request r's pages are
 *     page_table[page_off_r .. page_off_r + ceil(kv_len_r / P) - 1] with
 *     page_off_r = sum_{r' < r} ceil(kv_len_r' / P). Token j of request r is
 *     slot j % P of page page_table[page_off_r + j / P].
 *   - K and V pools: bf16 [num_pages][P][Hkv][D], row-major, separate buffers.
 *   - q / out: bf16 [sum qo_len][Hq][D] (requests packed in order); lse: fp32
 *     [sum qo_len][Hq], natural log of sum_j exp(s_j), s_j = sm_scale * q.k_j.
 *   - GQA: q head h reads kv head h / (Hq / Hkv).
 *   - Memory in the pools outside the request's keys (other pages, slots past
 *     kv_len in the last page) is never read into a result and may hold
 *     anything, NaN included.
 *
 * Ownership: the caller owns every device buffer (q, pools, page table, out,
 * lse, workspace); the library owns the plan (host memory plus a pinned host
 * copy of its work list, a block drawn from a library-owned pool when the
 * plan is made). Run calls are asynchronous on `stream` (a hipStream_t; NULL
 * means the null stream), allocate nothing, never synchronise the host, and
 * copy the plan's work list into the head of the workspace with a small
 * kernel that reads the plan's pinned block. The workspace must stay alive
 * until the stream has passed the call, and one workspace must not serve two
 * calls that can overlap. The plan may be destroyed as soon as the run calls
 * have returned: its pinned block goes back to the pool and is handed out
 * again only after the device has passed every upload that read it.
 *
 * Errors: every call returns a bia_status; nothing is thrown across the ABI.
 * Arguments are checked before anything is enqueued. bia_last_error() gives a
 * thread-local message for the last non-OK status on the calling thread.
 */
#ifndef BIA_H_
#define BIA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bia_status {
  BIA_OK = 0,
  BIA_ERR_INVALID_ARG = 1, /* null pointer, bad mode, bad split size, ...   */
  BIA_ERR_SHAPE = 2,       /* indptr not monotone, qo_len > kv_len, ...      */
  BIA_ERR_PAGE_RANGE = 3,  /* a page id outside [0, num_pages)               */
  BIA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the plan's   */
  BIA_ERR_UNSUPPORTED = 5, /* head_dim, page size or GQA group not built    */
  BIA_ERR_HIP = 6          /* a HIP runtime call failed                      */
} bia_status;

typedef enum bia_mode {
  BIA_MODE_PREFILL = 0, /* any qo_len_r in [0, kv_len_r]                   */
  BIA_MODE_DECODE = 1   /* qo_len_r == 1 for every request                 */
} bia_mode;

/* Default split-KV partition sizes (sglang PR #10417, Modifications). */
#define BIA_PREFILL_SPLIT 4096
#define BIA_DECODE_SPLIT 2048
/* Rows of the prefill q tile; rows are (token, head-in-group) pairs packed
 * token-major, so one tile holds 128 / (Hq / Hkv) tokens of one kv head. */
#define BIA_Q_TILE_ROWS 128
/* Keys per KV tile; a split size must be a positive multiple of it. */
#define BIA_KV_TILE 64
#define BIA_PAGE_SIZE 16

/* Plan flags. BIA_PLAN_STRICT_CHUNK_ALIGN: reject (BIA_ERR_INVALID_ARG) a
 * prefill request whose chunk does not start on the q-tile grid, i.e. whose
 * kv_len - qo_len is not a multiple of bia_prefill_chunk_align() tokens (the
 * startup rejection of a misaligned chunk size, sglang PR #43612, Summary). */
#define BIA_PLAN_STRICT_CHUNK_ALIGN 0x1u
/* Latent (MLA) plan: num_kv_heads 1 and head_dim 576 (512 latent + 64 rope
 * dims of the one cached row per token), values the first 512 of them; run it
 * with bia_mla_prefill_paged / bia_mla_decode_paged. */
#define BIA_PLAN_MLA 0x2u
#define BIA_MLA_QK_DIM 576
#define BIA_MLA_V_DIM 512
/* Largest split size of an MLA plan (the item's page list is held on chip). */
#define BIA_MLA_MAX_SPLIT 16384

typedef struct bia_plan bia_plan; /* opaque, library-owned */

/*
 * Build the work list of one prefill or decode call from the batch's lengths
 * alone (sglang PR #43612, Summary: the probe drives a paged prefill wrapper
 * planned with fixed_split_size; the split is a pure kernel knob).
 *
 *   qo_indptr, kv_indptr: host int32 [batch + 1], start at 0, non-decreasing,
 *       0 <= qo_len_r <= kv_len_r; in decode mode qo_len_r == 1.
 *   page_table: host int32 [sum ceil(kv_len_r / page_size)]; only checked
 *       (every id in [0, num_pages)); the run call reads the device copy,
 *       which must hold the same ids. May be NULL when no request has keys.
 *   num_qo_heads % num_kv_heads == 0 with a group of 1, 2, 4 or 8;
 *   head_dim 64 or 128; page_size 16;
 *   split_size > 0 and a multiple of BIA_KV_TILE (BIA_PREFILL_SPLIT /
 *       BIA_DECODE_SPLIT for the pages' setting). Keys of request r are cut
 *       into partitions [k * split_size, (k + 1) * split_size), anchored at
 *       key 0 of the request.
 *   flags: 0, BIA_PLAN_STRICT_CHUNK_ALIGN, BIA_PLAN_MLA or both. An MLA plan
 *       takes num_kv_heads 1, head_dim BIA_MLA_QK_DIM and num_qo_heads 8, 16,
 *       32, 64 or 128 (the one cached head is shared by every q head).
 * On success *out_plan receives a plan to free with bia_plan_destroy. The
 * arrays are not retained. batch == 0 gives an empty plan whose runs do
 * nothing. The pinned copy of the work list is taken here (from the pool, or
 * newly pinned with hipHostMalloc when no free block is large enough), so
 * run calls allocate nothing. In a process that sees no GPU the plan is made
 * without it: it can be inspected, and a run returns BIA_ERR_HIP.
 */
bia_status bia_plan_create(bia_mode mode, const int32_t* qo_indptr,
                           const int32_t* kv_indptr, const int32_t* page_table,
                           int32_t batch, int32_t num_qo_heads,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, int32_t num_pages,
                           int32_t split_size, uint32_t flags,
                           bia_plan** out_plan);

/* Bytes of device workspace a run of this plan needs (0 for NULL). */
size_t bia_plan_workspace_bytes(const bia_plan* plan);

/* Free a plan. Allowed as soon as the run calls made with it have returned,
 * also while their work is still queued: the pinned block goes back to the
 * library's pool without being freed and without waiting for the device.
 * NULL is a no-op. */
void bia_plan_destroy(bia_plan* plan);

/*
 * Causal prefill of a BIA_MODE_PREFILL plan (sglang PR #43612, Summary;
 * sglang PR #10417, Modifications).
 *   q: device bf16 [sum qo_len][Hq][D]; k_pool, v_pool: device bf16
 *   [num_pages][16][Hkv][D]; page_table_dev: device int32, same ids as the
 *   plan's; out: device bf16 [sum qo_len][Hq][D]; lse: device fp32
 *   [sum qo_len][Hq] or NULL to skip it; workspace: device, at least
 *   bia_plan_workspace_bytes(plan) bytes, 256-byte aligned.
 * Output bits of a request depend only on its q, its keys and values, its
 * qo_len, kv_len, split_size and sm_scale.
 */
bia_status bia_prefill_paged(const bia_plan* plan, const void* q,
                             const void* k_pool, const void* v_pool,
                             const int32_t* page_table_dev, float sm_scale,
                             void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Decode of a BIA_MODE_DECODE plan: one query token per request attends to
 * all kv_len_r keys (sglang PR #10417, Modifications: batch-invariant decode
 * with a fixed split of 2048).
 *   q, out: device bf16 [batch][Hq][D]; lse: device fp32 [batch][Hq] or NULL;
 *   other arguments as for bia_prefill_paged.
 */
bia_status bia_decode_paged(const bia_plan* plan, const void* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* page_table_dev, float sm_scale,
                            void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * bia_decode_paged for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same output bits, with the workspace
 * taken from a library-owned static device array of
 * BIA_STATIC_WORKSPACE_BYTES on each GPU instead of a caller buffer. The
 * caller still passes the plan, inputs and outputs (as for bia_decode_paged,
 * on the current device's stream); the call allocates nothing (the plan's
 * pinned work list was taken when the plan was made).
 *   BIA_ERR_WORKSPACE: bia_plan_workspace_bytes(plan) exceeds
 *   BIA_STATIC_WORKSPACE_BYTES (about 32 MiB holds a batch of 64 requests
 *   with contexts of up to 32768 tokens at 8 kv heads x 4 q heads, D 128).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero: each call writes its work
 * list and partial states before reading them). Calls that can overlap on
 * one GPU (on two streams, or from two threads) race on it and must not be
 * made.
 */
#define BIA_STATIC_WORKSPACE_BYTES (32u << 20)
bia_status bia_decode_paged_static(const bia_plan* plan, const void* q,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* page_table_dev, float sm_scale,
                                   void* out, float* lse, void* stream);

/*
 * Latent (MLA) attention over a paged latent cache, absorbed form: the MLA
 * decode path that the pages name as lacking a deterministic mode (sglang PR
 * #43612, Summary), given the same fixed-split, fixed-order treatment as the
 * calls above (sglang PR #10417, Modifications). Every q head scores its 576
 * dims against the one cached 576-dim row of each key and averages the first
 * 512 dims of those rows:
 *   out[t][h] = sum_j softmax_j(sm_scale * q[t][h] . kv[j]) kv[j][0:512]
 * over the keys j <= the token's position (causal; decode: all kv_len keys).
 *   plan: made with BIA_PLAN_MLA, of the call's mode;
 *   q: device bf16 [sum qo_len][Hq][576]; kv_pool: device bf16
 *   [num_pages][16][576]; out: device bf16 [sum qo_len][Hq][512]; lse: device
 *   fp32 [sum qo_len][Hq] or NULL; page_table_dev, workspace: as for
 *   bia_prefill_paged.
 * A plan without BIA_PLAN_MLA is rejected (BIA_ERR_INVALID_ARG), and so is an
 * MLA plan passed to bia_prefill_paged / bia_decode_paged /
 * bia_append_paged_kv. Output bits of a request depend only on its q, its
 * cached rows, qo_len, kv_len, split_size, Hq and sm_scale.
 */
bia_status bia_mla_prefill_paged(const bia_plan* plan, const void* q,
                                 const void* kv_pool, const int32_t* page_table_dev,
                                 float sm_scale, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);
bia_status bia_mla_decode_paged(const bia_plan* plan, const void* q,
                                const void* kv_pool, const int32_t* page_table_dev,
                                float sm_scale, void* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Merge partial attention states in a fixed order: row i folds states
 * state_indptr[i] .. state_indptr[i+1]-1 in ascending order. A state with
 * lse = -inf is empty and skipped; the rest combine as
 *   M = max lse_k, w_k = exp(lse_k - M), o = sum w_k o_k / sum w_k,
 *   lse = M + log sum w_k
 * (the fixed-order merge of split-KV partial states, sglang PR #10417,
 * Modifications). A row with only empty states gives o = 0, lse = -inf. The
 * prefill and decode calls fold their own partitions with the same function.
 *   v: device fp32 [n_states][num_heads][head_dim]; s: device fp32
 *   [n_states][num_heads]; state_indptr_dev: device int32 [n_rows + 1];
 *   out: device bf16 [n_rows][num_heads][head_dim]; out_lse: device fp32
 *   [n_rows][num_heads] or NULL. head_dim 64 or 128. The indptr is read on
 *   the device only and must start at 0 and be non-decreasing with its last
 *   entry <= n_states (not checked).
 */
bia_status bia_merge_states(const float* v, const float* s,
                            const int32_t* state_indptr_dev, int32_t n_rows,
                            int32_t num_heads, int32_t head_dim, void* out,
                            float* out_lse, void* stream);

/*
 * Write the keys and values of each request's qo_len new tokens into its
 * pages, before the attention call that reads them (the step ahead of a
 * chunked prefill or a decode over cached prefix pages, sglang PR #43612,
 * Summary). New token i of request r is KV position kv_len_r - qo_len_r + i,
 * slot (position % 16) of page page_table[page_off_r + position / 16].
 *   k_new, v_new: device bf16 [sum qo_len][Hkv][D], requests packed in order;
 *   k_pool, v_pool: device bf16 [num_pages][16][Hkv][D], written;
 *   page_table_dev, workspace: as for bia_prefill_paged (any plan mode).
 * Only the new tokens' slots are written; every other byte of the pools is
 * left as it was. Pages shared by two requests of one plan must not receive
 * new tokens of both (the writes would race).
 */
bia_status bia_append_paged_kv(const bia_plan* plan, const void* k_new,
                               const void* v_new, const int32_t* page_table_dev,
                               void* k_pool, void* v_pool, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Decode without host planning, for callers that replay it from a HIP graph
 * (a captured call holds no host-to-device copy and allocates nothing). The
 * pages' runtime turns split-KV off while capturing and replaying graphs
 * ("[POC] Support deterministic inference", sglang PR #10417, Modifications,
 * and the review thread on disable_split_kv), so its bits depend on whether
 * a graph ran; here the partitions stay at split_size in graph mode, and a
 * request's out / lse bits equal those of bia_decode_paged with a plan of
 * the same split_size.
 *
 * bia_decode_graph_create fixes the capacity: up to max_batch requests, each
 * with 1 <= kv_len <= max_kv_len, and page tables of up to
 * page_table_capacity entries. The other arguments are as for
 * bia_plan_create (head_dim 64 or 128, page_size 16, split_size a positive
 * multiple of 64). The handle is host memory owned by the library.
 *
 * bia_decode_graph_workspace_bytes: bytes of workspace a run needs (it holds
 * the per-request flags, the work list made on the device and the partial
 * states of up to ceil(max_kv_len / split_size) partitions per request and
 * kv head).
 *
 * bia_decode_graph_run: decode of `batch` requests (0 <= batch <= max_batch;
 * `batch` and every pointer are baked into a captured graph, the contents of
 * the buffers are not). kv_indptr_dev: device int32 [batch + 1], starting at
 * 0 (cumulative kv lengths, as kv_indptr of bia_plan_create); q, out: device
 * bf16 [batch][Hq][D]; lse: device fp32 [batch][Hq] or NULL; page_table_dev:
 * device int32 with request r's pages at page_off_r as for the other calls;
 * workspace: device, >= bia_decode_graph_workspace_bytes, 256-byte aligned.
 * Launches a planner kernel (one workgroup per request), the decode kernel
 * over batch * Hkv * ceil(max_kv_len / split_size) fixed slots (slots past a
 * request's partitions return at once) and, when a request can span more
 * than one partition, the fixed-order merge. Host-side checks run before
 * anything is enqueued; the device checks each request (1 <= kv_len <=
 * max_kv_len, its pages within page_table_capacity, every page id in
 * [0, num_pages)) and an invalid request reads no keys: its rows come out as
 * the empty state (o = 0, lse = -inf) and its flag is set.
 *
 * bia_decode_graph_read_flags: copies the flags of the last run on this
 * workspace to host int32 [batch] and waits for the stream (not for use
 * inside a captured region): 0 = valid, else a sum of 1 (kv_len outside
 * [1, max_kv_len]), 2 (pages past page_table_capacity), 4 (a page id outside
 * [0, num_pages)).
 */
typedef struct bia_decode_graph bia_decode_graph; /* opaque, library-owned */
bia_status bia_decode_graph_create(int32_t max_batch, int32_t num_qo_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t page_size, int32_t num_pages,
                                   int32_t max_kv_len, int32_t page_table_capacity,
                                   int32_t split_size, bia_decode_graph** out);
size_t bia_decode_graph_workspace_bytes(const bia_decode_graph* dg);
void bia_decode_graph_destroy(bia_decode_graph* dg);
bia_status bia_decode_graph_run(const bia_decode_graph* dg, int32_t batch,
                                const int32_t* kv_indptr_dev, const void* q,
                                const void* k_pool, const void* v_pool,
                                const int32_t* page_table_dev, float sm_scale,
                                void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);
bia_status bia_decode_graph_read_flags(const bia_decode_graph* dg,
                                       const void* workspace, int32_t batch,
                                       int32_t* flags_host, void* stream);

/* Chunk alignment, in tokens, under which a chunked prefill reproduces the
 * unchunked one bit for bit: 128 (the PREFILL_Q_TILE_TOKENS = 128 constant of
 * sglang PR #43612, Summary). Chunk starts that are multiples of it land on
 * the q-tile grid for every GQA group the library supports. */
int32_t bia_prefill_chunk_align(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* bia_last_error(void);

/* Host-side introspection of a plan's work list, for tests and tools.
 * bia_plan_num_items: number of compute work items (workgroups launched).
 * bia_plan_get_items: copies min(n, num_items) items of 8 int32 each:
 *   {q_row0, n_tok, pos0, kv_len, page_off, kv_head, kv_begin, state}
 *   in launch order (see the workspace layout in the library source).
 * bia_plan_num_states: partial (o, lse) states the plan writes before its
 *   merge (0 when every row has a single partition). */
int32_t bia_plan_num_items(const bia_plan* plan);
int32_t bia_plan_get_items(const bia_plan* plan, int32_t* items, int32_t n);
int64_t bia_plan_num_states(const bia_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* BIA_H_ */
