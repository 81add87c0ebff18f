// Batch- and chunk-invariant paged attention for gfx950 (MI355X, CDNA4):
// prefill, decode and state-merge kernels plus the C-ABI launch layer.
//
// Invariance rules every kernel here keeps (they make a row's bits a function
// of its own q, keys, values, lengths, split size and scale only):
//  1. Tile shapes and the kernel variant never depend on the batch.
//  2. KV tiles (64 keys) and split-KV partitions (a fixed multiple of 64) are
//     anchored at key 0 of the request, never at the chunk or the q tile
//     (fixed split-KV, sglang PR #10417, Modifications).
//  3. A key a row must not see is replaced by -inf before the softmax; the
//     arithmetic is otherwise the same for masked and unmasked tiles.
//  4. A tile with no visible key for a row is an exact no-op for that row:
//     its rescale factor is exactly 1 and its probabilities exactly 0.
//  5. Partial (o, lse) states of a row's partitions fold in ascending
//     partition order through one function (fold_state); empty states
//     (lse = -inf) are skipped.
//  6. Memory past a request's keys is never loaded into a product: those K/V
//     slots are zero-filled in registers/LDS.
//  7. Element offsets are 64-bit.
//  8. No atomics and no reduction whose order depends on scheduling.
// Rules 2-4 make a q row's arithmetic independent of which q tile holds it,
// which is what lets a chunked prefill on the 128-row grid reproduce the
// unchunked one (sglang PR #43612, Summary).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>
#include <algorithm>
#include <type_traits>

#include "bia.h"
#include "plan.h"

using bia::MergeItem;
using bia::WorkItem;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -INFINITY;
constexpr int kThreads = 256;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float a) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}

// ---------------------------------------------------------------------------
// Fixed-order fold of partial states (natural-log lse). Running state: M (max
// lse so far), sum (sum of exp(lse_k - M)), acc[i] (sum of exp(lse_k - M) *
// o_k[i]). Contraction is pinned by explicit fmaf so every inlined copy
// computes the same bits. One live state folds to exactly itself.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void fold_state(float& M, float& sum, float (&acc)[N],
                                           float lse_k, const float (&o_k)[N]) {
#pragma clang fp contract(off)
  if (lse_k == kNegInf) return;
  if (M == kNegInf) {
    M = lse_k;
    sum = 1.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = o_k[i];
  } else if (lse_k <= M) {
    const float w = fast_exp2((lse_k - M) * kLog2e);
    sum = sum + w;
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = __builtin_fmaf(w, o_k[i], acc[i]);
  } else {
    const float a = fast_exp2((M - lse_k) * kLog2e);
    sum = __builtin_fmaf(sum, a, 1.0f);
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = __builtin_fmaf(acc[i], a, o_k[i]);
    M = lse_k;
  }
}

// Final output of a fold: o = acc / sum, lse = M + ln(sum); empty -> (0, -inf).
template <int N>
__device__ __forceinline__ float fold_finish(float M, float sum, float (&acc)[N]) {
#pragma clang fp contract(off)
  if (M == kNegInf) {
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0f;
    return kNegInf;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = acc[i] / sum;
  return M + fast_log2(sum) * kLn2;
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup = one WorkItem = 128 q rows (128/g tokens x g heads
// of one kv head) over one split-KV partition. 4 waves x 32 rows. Per 64-key
// tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as M, q rows as N,
// head dim as K), so each lane holds 32 scores of ONE q row and the online
// softmax is per lane (plus one exchange with lane ^ 32); then O^T += V^T P^T
// with the probabilities straight from registers as the B operand.
//
// K and V reach LDS by DMA (global_load_lds_dwordx4: 16 bytes per lane from
// the lane's own global address into LDS at M0 + 16 * lane, checked on the
// GPU with an in-bounds probe), so no registers stage them. Two buffers each
// for K and V; per tile: wait for this wave's DMAs, one barrier, then the
// DMAs of K(j+2) and V(j+1) into the buffers the previous tile finished with
// (each wave issues its share after a different score MFMA, so the four
// waves' bursts do not queue behind each other), the score MFMAs of tile j+1
// overlapped with the softmax of tile j, then PV of tile j. The DMAs are
// inline asm with an explicit wait, so the
// compiler does not make every later LDS read wait for all outstanding loads.
//
// LDS rows are 2D bytes, unpadded (a DMA instruction fills 1 KB
// contiguously); the 16-byte slot of chunk c of row r is c ^ swz(r), which
// keeps 16 consecutive rows of one chunk (the K operand reads) and 4
// consecutive rows of 2 chunks (the transposing V reads) on distinct banks.
// The V^T operand comes from ds_read_b64_tr_b16: in each 16-lane group, lane
// i addresses 4 dims of key i / 4 and lane j = 4a + b receives dim 4a + b of
// those 4 keys.
//
// MFMA 32x32x16 layouts (lane l, hi = l / 32, c = l % 32): A[m][k]: m = c,
// k = 8 hi + e; B[k][n]: n = c, k = 8 hi + e; D[m][n]: n = c,
// m = 8 (v / 4) + 4 hi + v % 4. The PV contraction uses the key order in
// which the score MFMA left the probabilities in registers: slot 8 hi + e of
// (key block kb, half h) is key 32 kb + 16 h + 8 (e / 4) + 4 hi + e % 4; V^T
// is read in the same order.
//
// Softmax bookkeeping, all per row and so independent of the tile holding
// the row: the running max m is raised only when a tile's max exceeds it by
// more than kLazyMax (base-2 units), so most tiles rescale nothing, and the
// tile max is only taken when a lane's probability sum against the current m
// exceeds 2^kLazyMax (or on the row's first tile with a visible key); scores
// are scaled inside the exponent (exp2(s * c - m)); masking runs only on
// tiles that reach past the wave's first row position (elsewhere every key
// is visible to every row of the wave). The row sum adds the fp32
// probabilities (summing their bf16 roundings would cost ~1e-3 in lse).
// ---------------------------------------------------------------------------
constexpr float kLazyMax = 8.0f;
constexpr float kLazyP = 256.0f;  // 2^kLazyMax

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* p) {
  // p points into __shared__ memory; the C-style cast moves it to the LDS
  // address space, which the transposing read requires.
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Byte offset of a __shared__ address within the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) const char*)(p)));
}

// 16 bytes from this lane's global address to LDS byte lds_base + 16 * lane;
// lds_base must be the same on every lane of the wave.
__device__ __forceinline__ void lds_dma16(const void* gaddr, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(base)
               : "memory");
}

__host__ __device__ constexpr uint64_t join_u64(uint32_t hi, uint32_t lo) {
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
static_assert(join_u64(0x00007f12u, 0x80004000u) == 0x00007f1280004000ull,
              "64-bit address widening must not sign-extend the low word");

// Same, with the global address split into a wave-uniform 64-bit base (an
// SGPR pair) and this lane's 32-bit byte offset from it.
__device__ __forceinline__ void lds_dma16_sbase(uint32_t lane_off, const void* base,
                                                uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  // readfirstlane returns int: each half goes through uint32_t, or the low
  // half would sign-extend into the high word.
  const uint64_t sb = join_u64(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
                                   static_cast<uint32_t>(b >> 32))),
                               static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
                                   static_cast<uint32_t>(b))));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_off), "s"(sb), "s"(m0)
               : "memory");
}

// N DMA instructions sharing one M0: instruction r reads global
// (base - 1024 r) + off[r] + 1024 r = base + off[r] and writes LDS
// m0 + 1024 r + 16 lane (the immediate offset moves both addresses).
template <int N>
__device__ __forceinline__ void dma_page(const uint32_t (&off)[N], uint64_t base, uint32_t m0) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(m0);
  uint64_t sb[N];
#pragma unroll
  for (int r = 0; r < N; ++r) {
    const uint64_t b = base - 1024ull * r;
    sb[r] = join_u64(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
                         static_cast<uint32_t>(b >> 32))),
                     static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b))));
  }
  if constexpr (N == 4) {
    asm volatile(
        "s_mov_b32 m0, %8\n\t"
        "global_load_lds_dwordx4 %0, %4\n\t"
        "global_load_lds_dwordx4 %1, %5 offset:1024\n\t"
        "global_load_lds_dwordx4 %2, %6 offset:2048\n\t"
        "global_load_lds_dwordx4 %3, %7 offset:3072"
        :
        : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(sb[0]), "s"(sb[1]),
          "s"(sb[2]), "s"(sb[3]), "s"(m)
        : "memory");
  } else {
    static_assert(N == 2, "2 or 4 instructions per page");
    asm volatile(
        "s_mov_b32 m0, %4\n\t"
        "global_load_lds_dwordx4 %0, %2\n\t"
        "global_load_lds_dwordx4 %1, %3 offset:1024"
        :
        : "v"(off[0]), "v"(off[1]), "s"(sb[0]), "s"(sb[1]), "s"(m)
        : "memory");
  }
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// max over lanes l and l ^ 32
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(x, fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(r[0])),
                        __builtin_bit_cast(float, static_cast<unsigned>(r[1]))));
}

// Slot permutation of a row (a bijection on the row's 16-byte slots).
// D = 128 (16 slots): 16 consecutive rows at one chunk take 16 distinct
// slots (the K operand reads), and rows 4q..4q+3 at chunks 4b..4b+3 take 16
// distinct slots (a transposing V read by 32 lanes).
template <int D>
__device__ __forceinline__ int lds_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 1) | ((r >> 2) & 1);
}

#ifndef BIA_PREFILL_MIN_BLOCKS
#define BIA_PREFILL_MIN_BLOCKS 2
#endif

template <int D>
__global__ void __launch_bounds__(kThreads, BIA_PREFILL_MIN_BLOCKS)
prefill_kernel(const WorkItem* __restrict__ items, const uint16_t* __restrict__ q,
               const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
               const int32_t* __restrict__ page_table, float scale_log2,
               int num_qo_heads, int num_kv_heads, int group_shift, int split,
               uint16_t* __restrict__ out, float* __restrict__ lse_out,
               float* __restrict__ o_part, float* __restrict__ lse_part) {
  constexpr int RB = D * 2;            // bytes per K/V row in LDS
  constexpr int SLOTS = D / 8;         // 16-byte slots per row
  constexpr int RPI = 1024 / RB;       // rows one DMA instruction fills (4 or 8)
  constexpr int IPW = 64 / (RPI * 4);  // DMA instructions per wave per tile and tensor
  constexpr int TB = 64 * RB;          // bytes per tile buffer
  constexpr int DB = D / 32;           // 32-wide d blocks of the output
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * TB];  // K0 K1 V0 V1

  const WorkItem it = items[blockIdx.x];
  if (it.n_tok == 0) return;  // padding of the XCD-interleaved launch order
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int hi = lane >> 5;
  const int col = lane & 31;
  const int g = 1 << group_shift;
  const int x = wave * 32 + col;  // this lane's row of the q tile
  const int tok = x >> group_shift;
  const int hj = x & (g - 1);
  const bool row_valid = tok < it.n_tok;
  const int pos = row_valid ? it.pos0 + tok : -1;
  // the row has visible keys in this item's partition (its first tile holds one)
  const bool row_live = pos >= it.kv_begin;
  // Position of the wave's first row: tiles ending at or before it need no mask.
  const int wave_pos0 = it.pos0 + ((wave * 32) >> group_shift);
  const int64_t q_off =
      (static_cast<int64_t>(it.q_row0 + tok) * num_qo_heads + it.kv_head * g + hj) * D;

  bf16x8 qf[D / 16];  // loaded after the first page ids (prologue)

  const int last = it.pos0 + it.n_tok - 1;
  const int kv_end = min(it.kv_begin + split, last + 1);
  const int n_tiles = (kv_end - it.kv_begin + 63) >> 6;
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * D;
  const int64_t head_off = static_cast<int64_t>(it.kv_head) * D;
  const int32_t* pt = page_table + it.page_off;
  const uint32_t lds_base = lds_offset(lds);

  // ---- DMA of one tile of K or V (wave's share: IPW instructions) ----
  // Instruction r of this wave fills rows row0 .. row0 + RPI - 1 (one page),
  // row0 = RPI * (4 r + wave); lane l takes row row0 + l / SLOTS and puts its
  // 16 bytes in slot l % SLOTS, i.e. chunk (l % SLOTS) ^ swz(row).
  // Page ids of tile t (its 4 pages) as one vector load, lane l holding page
  // l % 4 (clamped to the item's last page, so the read is always in range;
  // a page past kv_end is never used). Vector rather than scalar loads: a
  // scalar load in flight would make every LDS wait of the tile wait for it
  // too (the two share a counter, and scalar loads return out of order); the
  // ids are taken out with readlane only when the tile's DMAs are issued, one
  // or two tiles later.
  const int last_page = (kv_end - 1) >> 4;
  auto pages = [&](int t) -> int32_t {
    return pt[min(((it.kv_begin + 64 * t) >> 4) + (lane & 3), last_page)];
  };
  auto page_id = [&](int32_t pgv, int r) -> int32_t {
    return __builtin_amdgcn_readlane(pgv, (RPI * (4 * r + wave)) >> 4);
  };
  // The page ids one wave's DMAs of a tile use, in SGPRs. They are taken out
  // of the vectors before any DMA of the step is issued and pinned there: the
  // DMAs are inline asm that the compiler does not count as loads, so a
  // page-id read placed after them gets a wait on the load counter that would
  // also wait for the DMAs just issued (a memory round trip every tile).
  struct TilePages {
    int32_t id[IPW];  // ragged tiles: page of DMA instruction r
    int32_t own;      // full tiles: page `wave` of the tile
  };
  auto take_pages = [&](int32_t pgv) -> TilePages {
    TilePages tp;
#pragma unroll
    for (int r = 0; r < IPW; ++r) {
      tp.id[r] = page_id(pgv, r);
      asm volatile("" : "+s"(tp.id[r]));
    }
    tp.own = __builtin_amdgcn_readlane(pgv, wave);
    asm volatile("" : "+s"(tp.own));
    return tp;
  };
  // Full tiles: wave w fills rows 16 w .. 16 w + 15 (page w of the tile);
  // instruction r covers rows 16 w + RPI r + lane / SLOTS. All IPW
  // instructions share one M0 (the wave's 1 KB x IPW of the buffer) and
  // differ in the immediate offset 1024 r, which moves the LDS destination
  // and the global address alike, so the global base of instruction r is
  // taken back by the same amount. A lane's byte offset from the page base
  // is fixed per instruction for the whole kernel (the swizzle makes it
  // depend on r). One M0 write per tile and tensor instead of one per DMA.
  uint32_t dma_off[IPW];
#pragma unroll
  for (int r = 0; r < IPW; ++r) {
    const int row = RPI * r + lane / SLOTS;  // row within the page
    dma_off[r] = static_cast<uint32_t>(
        (row * slot_stride + head_off + ((lane % SLOTS) ^ lds_swz<D>(16 * wave + row)) * 8) * 2);
  }
  auto issue = [&](const uint16_t* __restrict__ pool, int t, int buf, const TilePages& tp) {
    const int t0 = it.kv_begin + 64 * t;
    if (t0 + 64 <= kv_end) {  // uniform: every row of the tile is a key of the item
      const uint64_t page_base = reinterpret_cast<uint64_t>(
          pool + static_cast<int64_t>(tp.own) * 16 * slot_stride);
      const uint32_t m0 = lds_base + buf * TB + wave * 16 * RB;
      dma_page<IPW>(dma_off, page_base, m0);
    } else {
#pragma unroll
      for (int r = 0; r < IPW; ++r) {
        const int row0 = RPI * (4 * r + wave);
        const int row = row0 + lane / SLOTS;
        const int chunk = (lane % SLOTS) ^ lds_swz<D>(row);
        const int key = t0 + row;
        const int dst = buf * TB + row0 * RB;
        if (key < kv_end) {
          const uint16_t* src = pool + (static_cast<int64_t>(tp.id[r]) * 16 + (key & 15)) *
                                           slot_stride + head_off + chunk * 8;
          lds_dma16(src, lds_base + dst);
        } else {  // past the item's keys: zero, never stale LDS contents
          *reinterpret_cast<uint4*>(&lds[dst + lane * 16]) = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  // K operand: row 32 kb + col, chunk 2 s + hi (16 bytes of dims 16 s + 8 hi ..).
  const int k_sw = lds_swz<D>(col);
  auto scores = [&](f32x16 (&acc)[2], int buf) {
    const uint8_t* kb = &lds[buf * TB + col * RB];
    acc[0] = f32x16{};
    acc[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int slot = (2 * s + hi) ^ k_sw;
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        const uint4 kw = *reinterpret_cast<const uint4*>(kb + 32 * kbk * RB + slot * 16);
        acc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kw),
                                                           qf[s], acc[kbk], 0, 0, 0);
      }
    }
  };
  // V^T operand (transposing reads): in 16-lane group G = lane / 16 (hi = G / 2,
  // dims 16 (G % 2) ..), lane i = lane % 16 addresses key kq = i / 4 of the
  // 4-key run and dims 4 (i % 4) .. + 3; the second read of an MFMA is 8 keys on.
  const int vq = (lane & 15) >> 2;
  const int v_lo = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within a 32-dim block
  const int v_byte = (lane & 1) * 8;
  int v_row_off[2], v_sw[2];
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) {
    const int r = 4 * hi + 8 * e2 + vq;  // row modulo 16 (32 kb + 16 h do not change swz)
    v_row_off[e2] = r * RB + v_byte;
    v_sw[e2] = lds_swz<D>(r);
  }

  float m = kNegInf;  // running max (base-2 scaled logits), possibly stale by < kLazyMax
  float lsum = 0.0f;  // this lane-half's running sum of probabilities
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};

  // ---- prologue: K(0), V(0), K(1) by DMA; scores of tile 0 ----
  f32x16 sacc[2];
  int32_t pg_v = pages(0);
  int32_t pg_k = pages(1);
  // q after the page ids: the first DMAs wait only for the ids, and the q
  // tile's latency overlaps theirs
  // (rows past the tile's tokens read the tile's first token instead: an
  // unconditional load, and those rows are never written)
  const int64_t q_ld = row_valid ? q_off
                                 : (static_cast<int64_t>(it.q_row0) * num_qo_heads +
                                    it.kv_head * g + hj) * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + q_ld + 16 * s + 8 * hi));
  {
    const TilePages p0 = take_pages(pg_v);
    const TilePages p1 = take_pages(pg_k);
    issue(kp, 0, 0, p0);
    issue(vp, 0, 2, p0);
    if (n_tiles > 1) issue(kp, 1, 1, p1);
  }
  pg_v = pg_k;
  pg_k = pages(2);
  wait_dma();
  __syncthreads();
  scores(sacc, 0);

  // One tile: wait + barrier, DMAs of K(j+2) and V(j+1), score MFMAs of tile
  // j+1 (into nxt) overlapped with the softmax of tile j (cur), PV of tile j.
  // P is the parity of j (K(j+1) is in buffer 1 - P, V(j) in buffer 2 + P).
  // K fragment of score MFMA i (head-dim step i / 2, key block i % 2).
  // Per-lane offsets of K step s = 2 a + c: kbase[c] ^ 64 a, since chunk
  // (2 s + hi) ^ swz = (4 a) ^ ((2 c + hi) ^ swz); of the V^T reads of d block
  // b: vbase[e2] ^ 64 b, since (4 b + v_lo) ^ swz = (4 b) ^ (v_lo ^ swz). Two
  // registers each instead of eight; bits 6-7 of these offsets hold nothing
  // else (row * RB is a multiple of 256, v_byte is 0 or 8).
  uint32_t kbase[2], vbase[2];
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    kbase[c2] = static_cast<uint32_t>(col * RB + (((2 * c2 + hi) ^ k_sw) * 16));
    vbase[c2] = static_cast<uint32_t>(v_row_off[c2] + ((v_lo ^ v_sw[c2]) * 16));
  }
  auto kfrag = [&](int buf, int i) -> bf16x8 {
    const int s2 = i >> 1;
    const uint32_t off = kbase[s2 & 1] ^ static_cast<uint32_t>(64 * (s2 >> 1));
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(&lds[buf * TB + (32 * (i & 1)) * RB + off]));
  };
  // V^T fragment of PV MFMA i: key block kb = i / (2 DB), half h = (i / DB) % 2,
  // dim block b = i % DB (so consecutive MFMAs accumulate into different o[b]).
  auto vfrag = [&](int buf, int i) -> bf16x8 {
    const int b = i % DB;
    const int kbk = i / (2 * DB);
    const int h = (i / DB) & 1;
    const uint8_t* rb = &lds[buf * TB + (32 * kbk + 16 * h) * RB];
    const uint2 lo = lds_read_tr16(rb + (vbase[0] ^ static_cast<uint32_t>(64 * b)));
    const uint2 up = lds_read_tr16(rb + (vbase[1] ^ static_cast<uint32_t>(64 * b)));
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, up.x, up.y));
  };

  // One tile: wait + barrier; DMAs of K(j+2) and V(j+1) into the buffers the
  // previous tile finished with; phase A: the 16 score MFMAs of tile j+1 (into
  // nxt) hand-interleaved with the softmax of tile j (cur), K reads two MFMAs
  // ahead; phase B: the PV MFMAs of tile j, V reads two MFMAs ahead. Each
  // group ends in a scheduling fence so the compiler keeps the interleave.
  // P is the parity of j (K(j+1) is in buffer 1 - P, V(j) in buffer 2 + P).
  auto body = [&](auto has_next, auto parity, f32x16 (&cur)[2], f32x16 (&nxt)[2], int j) {
    constexpr bool kHasNext = decltype(has_next)::value;
    constexpr int P = decltype(parity)::value;
    wait_dma();
    __syncthreads();  // K(j+1), V(j) are in LDS; every wave is done with tile j-1
    // the derived offsets are recomputed per tile rather than kept live
    // (kept live, they and the page ids below push the loop into spills)
    asm volatile("" : "+v"(kbase[0]), "+v"(kbase[1]), "+v"(vbase[0]), "+v"(vbase[1]));
    // Page ids right after the barrier. For whole tiles (K(j+2) whole implies
    // V(j+1) whole) the DMAs go out later, after score MFMA wave * D / 32 of
    // phase A, so the four waves' bursts reach the address path one after
    // another instead of all right after the barrier; each wave then needs
    // only its own page of each tile. Ragged tiles go out at once.
    bool stagger = false;
    int32_t own_k = 0, own_v = 0;
    if constexpr (kHasNext) {
      stagger = it.kv_begin + 64 * (j + 3) <= kv_end;
      if (stagger) {
        own_k = __builtin_amdgcn_readlane(pg_k, wave);
        own_v = __builtin_amdgcn_readlane(pg_v, wave);
        asm volatile("" : "+s"(own_k), "+s"(own_v));
      } else {
        const TilePages kpg = take_pages(pg_k);
        const TilePages vpg = take_pages(pg_v);
        if (j + 2 < n_tiles) issue(kp, j + 2, P, kpg);
        issue(vp, j + 1, 3 - P, vpg);
      }
      pg_v = pg_k;
      pg_k = pages(j + 3);
    }
    auto dmas = [&]() {
      if (!stagger) return;
      dma_page<IPW>(dma_off,
                    reinterpret_cast<uint64_t>(kp + static_cast<int64_t>(own_k) * 16 * slot_stride),
                    lds_base + P * TB + wave * 16 * RB);
      dma_page<IPW>(dma_off,
                    reinterpret_cast<uint64_t>(vp + static_cast<int64_t>(own_v) * 16 * slot_stride),
                    lds_base + (3 - P) * TB + wave * 16 * RB);
    };
    const int t0 = it.kv_begin + 64 * j;
    if (t0 + 63 > wave_pos0) {  // wave-uniform: some key is past some row
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = t0 + 32 * kbk + 8 * (v >> 2) + 4 * hi + (v & 3);
          cur[kbk][v] = key <= pos ? cur[kbk][v] : kNegInf;
        }
      }
    }

    // The item's first tile: every row with a visible key has no max yet, so
    // below it would ask for the tile max and recompute its probabilities
    // (lsum and O, still zero, scaled by zero). The max is taken here instead,
    // as that path takes it, and the probabilities are computed once: the
    // same values, sums and order, so the same bits.
    if (j == 0) {
      float xm = cur[0][0];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int v = 0; v < 16; ++v) xm = fmaxf(xm, cur[kbk][v]);
      const float mt = max_halves(xm) * scale_log2;
      if (row_live && mt > m + kLazyMax) m = mt;  // m is -inf here
    }

    // ---- phase A ----
    // Probabilities against the running max as it stands, p = exp2(s c - m),
    // one key pair per score MFMA. With the lazy max no p exceeds
    // 2^kLazyMax unless the tile must raise m, and a lane's sum over its 32
    // keys exceeds 2^kLazyMax whenever one of its p does; so the tile max is
    // taken only when that sum (or a row with no max yet) asks for it.
    const float neg_m = (m == kNegInf) ? 0.0f : -m;
    float psum = 0.0f;
    uint32_t pw[16];  // packed bf16 probabilities, pair pi = 8 kb + (v / 2)
    // Software-pipelined by one pair: step pi takes the exponentials of pair
    // pi and sums and packs pair pi - 1, so no step waits on its own exp2
    // results. Step 16 only finishes pair 15. Same operations, same order.
    float e0 = 0.0f, e1 = 0.0f;
    auto softmax_step = [&](int pi) {
      if (pi > 0) {
        psum += e0;
        psum += e1;
        pw[pi - 1] = pack_bf16x2(e0, e1);
        asm volatile("" : "+v"(pw[pi - 1]), "+v"(psum));
      }
      if (pi < 16) {
        const int kbk = pi >> 3, v = 2 * (pi & 7);
        e0 = fast_exp2(__builtin_fmaf(cur[kbk][v], scale_log2, neg_m));
        e1 = fast_exp2(__builtin_fmaf(cur[kbk][v + 1], scale_log2, neg_m));
        asm volatile("" : "+v"(e0), "+v"(e1));
      }
    };
    if constexpr (kHasNext) {
      nxt[0] = f32x16{};
      nxt[1] = f32x16{};
      bf16x8 kf[3];
      kf[0] = kfrag(1 - P, 0);
      kf[1] = kfrag(1 - P, 1);
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        nxt[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % 3], qf[i >> 1], nxt[i & 1],
                                                             0, 0, 0);
        if (i + 2 < D / 8) kf[(i + 2) % 3] = kfrag(1 - P, i + 2);
        if (i < 16) softmax_step(i);
        if (i % (D / 32) == 0 && i / (D / 32) == wave) dmas();  // slot wave * D / 32
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = D / 8; i <= 16; ++i) softmax_step(i);
    } else {
#pragma unroll
      for (int i = 0; i <= 16; ++i) softmax_step(i);
    }

    // Raise test, per row. A row asks for it when either half's sum exceeds
    // 2^kLazyMax or it has visible keys in this partition and no max yet;
    // then it raises iff the tile max exceeds m by more than kLazyMax, and a
    // raised row recomputes its p. A row that does not raise keeps the p
    // above and alpha == 1 exactly, so its bits never depend on the other
    // rows of the wave.
    const bool ask = (psum > kLazyP) || (m == kNegInf && row_live);
    bool raise = false;
    float m_new = m, alpha = 1.0f;
    if (__any(ask)) {
      const auto sw = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(ask),
                                                       static_cast<unsigned>(ask), false, false);
      const bool ask_row = (static_cast<unsigned>(sw[0]) | static_cast<unsigned>(sw[1])) != 0u;
      float x = cur[0][0];
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int v = 0; v < 16; ++v) x = fmaxf(x, cur[kbk][v]);
      const float mt = max_halves(x) * scale_log2;
      raise = ask_row && mt > m + kLazyMax;  // true on a row's first tile with a visible key
      m_new = raise ? mt : m;
      alpha = raise ? fast_exp2(m - m_new) : 1.0f;
      if (__any(raise)) {
        const float neg_m2 = -m_new;  // finite wherever it is used (raise)
        float ps2 = 0.0f;
#pragma unroll
        for (int pi = 0; pi < 16; ++pi) {
          const int kbk = pi >> 3, v = 2 * (pi & 7);
          const float p0 = fast_exp2(__builtin_fmaf(cur[kbk][v], scale_log2, neg_m2));
          const float p1 = fast_exp2(__builtin_fmaf(cur[kbk][v + 1], scale_log2, neg_m2));
          ps2 += p0;
          ps2 += p1;
          const uint32_t w = pack_bf16x2(p0, p1);
          pw[pi] = raise ? w : pw[pi];
        }
        psum = raise ? ps2 : psum;
        lsum *= alpha;  // lanes that did not raise have alpha == 1 exactly
#pragma unroll
        for (int b = 0; b < DB; ++b) o[b] *= alpha;
      }
    }
    lsum += psum;
    m = m_new;

    // ---- phase B: O^T += V^T P^T (V of tile j, buffer 2 + P) ----
    constexpr int NPV = 4 * DB;
    bf16x8 vf[3];
    vf[0] = vfrag(2 + P, 0);
    vf[1] = vfrag(2 + P, 1);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int b = i % DB;
      const int pb0 = 4 * (i / DB);  // first pair of (kb, h)
      const uint4 pb = make_uint4(pw[pb0], pw[pb0 + 1], pw[pb0 + 2], pw[pb0 + 3]);
      o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % 3], __builtin_bit_cast(bf16x8, pb),
                                                     o[b], 0, 0, 0);
      if (i + 2 < NPV) vf[(i + 2) % 3] = vfrag(2 + P, i + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Unrolled by two so the score registers alternate without copies and the
  // buffer parity is a constant; the last tile has no successor.
  using T = std::true_type;
  using F = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  f32x16 sb[2];
  int j = 0;
  for (; j + 2 < n_tiles; j += 2) {
    body(T{}, P0{}, sacc, sb, j);
    body(T{}, P1{}, sb, sacc, j + 1);
  }
  if (j + 1 < n_tiles) {
    body(T{}, P0{}, sacc, sb, j);
    body(F{}, P1{}, sb, sacc, j + 1);
  } else {
    body(F{}, P0{}, sacc, sb, j);
  }

  // ---- this partition's state for the row: o = O / l, lse = m + log l ----
  // l: this lane's half plus lane ^ 32's (v_permlane32_swap hands each lane
  // its own and its partner's value; the sum is the same in either order)
  const auto lsw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, lsum),
                                                    __builtin_bit_cast(unsigned, lsum), false,
                                                    false);
  const float l_row = __builtin_bit_cast(float, static_cast<unsigned>(lsw[0])) +
                      __builtin_bit_cast(float, static_cast<unsigned>(lsw[1]));
  // The row's indices again, from a fresh lane id: kept live across the
  // tile loop they would take registers the loop needs.
  const int lane_e = static_cast<int>(
      __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
  const int hi_e = lane_e >> 5;
  const int x_e = wave * 32 + (lane_e & 31);
  const int tok_e = x_e >> group_shift;
  const int hj_e = x_e & (g - 1);
  float lse_nat = kNegInf;
  float inv = 0.0f;
  if (l_row > 0.0f) {
    inv = 1.0f / l_row;
    lse_nat = (m + fast_log2(l_row)) * kLn2;
  }
  if (it.state < 0) {
    // Whole rows out: the wave's 32 bf16 rows go to its quarter of the two K
    // buffers (no wave reads them after the last tile's barrier), 16-byte
    // chunk c of row r at slot c ^ (r % SLOTS); then each instruction stores
    // 1 KB of whole rows (RB bytes per row), the rows of one token's heads
    // being adjacent in `out`. One wave writes and reads its own region, so
    // LDS order within the wave suffices.
    uint8_t* stage = &lds[wave * 32 * RB];
    const int r_e = lane_e & 31;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int slot = (4 * b + v4) ^ (r_e & (SLOTS - 1));
        *reinterpret_cast<uint2*>(stage + r_e * RB + slot * 16 + hi_e * 8) =
            make_uint2(pack_bf16x2(o[b][4 * v4] * inv, o[b][4 * v4 + 1] * inv),
                       pack_bf16x2(o[b][4 * v4 + 2] * inv, o[b][4 * v4 + 3] * inv));
      }
    }
    constexpr int kRowsPerStore = 1024 / RB;
    constexpr int kStores = 32 / kRowsPerStore;
    const int c = lane_e % SLOTS;
    uint4 w[kStores];
#pragma unroll
    for (int i = 0; i < kStores; ++i) {
      const int rr = i * kRowsPerStore + lane_e / SLOTS;
      w[i] = *reinterpret_cast<const uint4*>(stage + rr * RB + (c ^ (rr & (SLOTS - 1))) * 16);
    }
    // all reads issued before the first store (else each is sunk into its
    // store's branch and waited for alone)
#pragma unroll
    for (int i = 0; i < kStores; ++i)
      asm volatile("" : "+v"(w[i].x), "+v"(w[i].y), "+v"(w[i].z), "+v"(w[i].w));
#pragma unroll
    for (int i = 0; i < kStores; ++i) {
      const int xr = wave * 32 + i * kRowsPerStore + lane_e / SLOTS;
      const int tr = xr >> group_shift;
      if (tr < it.n_tok)
        *reinterpret_cast<uint4*>(out + (static_cast<int64_t>(it.q_row0 + tr) * num_qo_heads +
                                         it.kv_head * g + (xr & (g - 1))) * D + c * 8) = w[i];
    }
    if (lse_out != nullptr && hi_e == 0 && tok_e < it.n_tok)
      lse_out[static_cast<int64_t>(it.q_row0 + tok_e) * num_qo_heads + it.kv_head * g + hj_e] = lse_nat;
  } else {
    if (tok_e >= it.n_tok) return;
    const int64_t st = static_cast<int64_t>(it.state) + x_e;
    float* orow = o_part + st * D;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d = 32 * b + 8 * v4 + 4 * hi_e;
        *reinterpret_cast<float4*>(orow + d) =
            make_float4(o[b][4 * v4] * inv, o[b][4 * v4 + 1] * inv, o[b][4 * v4 + 2] * inv,
                        o[b][4 * v4 + 3] * inv);
      }
    }
    if (hi_e == 0) lse_part[st] = lse_nat;
  }
}

// ---------------------------------------------------------------------------
// Decode on the VALU (head_dim 64, and splits past the MFMA decode's page
// list; head_dim 128 runs decode_mfma_kernel below): one workgroup = one
// WorkItem = (request, kv head, partition of up to `split` keys), g q heads. The partition's keys go in 16-key chunks to the 4
// waves round-robin (chunk c -> wave c % 4). In a wave, 8 lanes share one key
// (each holds D/8 of its dims, so 16-byte loads read whole rows) and a lane
// group takes keys c*16 + ks and c*16 + 8 + ks (one page). Chunks rotate
// through kDecodeBuffers (3) register buffers: the loads of a wave's next two
// chunks are in flight while the current one is computed, and page ids
// (scalar loads: a chunk is one page) are read a chunk earlier still.
//
// Scores: v_dot2_f32_bf16 partial dots, reduced over the 8 lanes with three
// DPP adds. PV: the two keys' probabilities (bf16) and the two keys' values
// of one dim form one v_dot2_f32_bf16, so each dim costs one instruction per
// key pair. Each 8-lane key group keeps its own online-softmax state (running
// max raised only past kLazyMax, rescale skipped when no lane raised); the
// groups, then the waves, combine in a fixed order at the end.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dpp_sum8(float x) {
#pragma clang fp contract(off)
  x = x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                        0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x = x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                        0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x = x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                        0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}

// Value of lane ^ 8 (within each 16-lane row).
__device__ __forceinline__ float dpp_ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x128, 0xF, 0xF, false));
}

// {x of this lane, x of lane ^ 16} (step 0) or {.., lane ^ 32} (step 1), in
// an order that depends on the lane.
__device__ __forceinline__ void lane_swap(int step, float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  if (step == 0) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
    b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
    b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
  }
}

// Symmetric combine of two base-2 online-softmax states (same result on both
// lanes of a butterfly pair: every term is computed the same way and the
// additions commute).
template <int N>
__device__ __forceinline__ void combine_sym(float& m, float& l, float (&o)[N], float m2, float l2,
                                            const float (&o2)[N]) {
#pragma clang fp contract(off)
  const float mm = fmaxf(m, m2);
  const float msub = (mm == kNegInf) ? 0.0f : mm;
  const float a = fast_exp2(m - msub);
  const float b = fast_exp2(m2 - msub);
  l = l * a + l2 * b;
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] = o[i] * a + o2[i] * b;
  m = mm;
}

// Chunks in flight per wave plus one (three register buffers), and the
// workgroups per CU the registers allow: two up to 4 q heads per kv head; at
// 8 the accumulators alone take 8 * D / 8 registers a lane, so one workgroup
// per CU keeps everything in registers (two would spill to scratch).
template <int G>
constexpr int kDecodeBuffers = 3;
template <int G>
constexpr int kDecodeBlocksPerCU = G <= 4 ? 2 : 1;

template <int D, int G>
__global__ void __launch_bounds__(kThreads, kDecodeBlocksPerCU<G>)
decode_kernel(const WorkItem* __restrict__ items, const uint16_t* __restrict__ q,
              const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
              const int32_t* __restrict__ page_table, float scale_log2, int num_qo_heads,
              int num_kv_heads, int split, uint16_t* __restrict__ out,
              float* __restrict__ lse_out, float* __restrict__ o_part,
              float* __restrict__ lse_part) {
  constexpr int DPL = D / 8;   // dims per lane
  constexpr int W = DPL / 2;   // packed bf16 pairs per lane
  constexpr int U = W / 4;     // 16-byte loads per lane per row
  constexpr int CHUNK = 16;    // keys per wave per chunk
  __shared__ float sm_ml[4][G][2];
  __shared__ float sm_o[4][G][D];

  const WorkItem it = items[blockIdx.x];
  if (it.n_tok == 0) return;  // a fixed-capacity slot past the request's partitions
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int ks = lane >> 3;    // key slot of this lane's group
  const int part = lane & 7;   // which D/8 dims of the key this lane holds

  uint32_t qw[G][W];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint16_t* qrow =
        q + (static_cast<int64_t>(it.q_row0) * num_qo_heads + it.kv_head * G + j) * D + part * DPL;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint4 w = *reinterpret_cast<const uint4*>(qrow + 8 * u);
      qw[j][4 * u] = w.x;
      qw[j][4 * u + 1] = w.y;
      qw[j][4 * u + 2] = w.z;
      qw[j][4 * u + 3] = w.w;
    }
  }

  const int kv_end = min(it.kv_begin + split, it.kv_len);
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * D;
  const int64_t head_off = static_cast<int64_t>(it.kv_head) * D + part * DPL;
  const int32_t* pt = page_table + it.page_off;
  float m[G], l[G], o[G][DPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNegInf;
    l[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[j][i] = 0.0f;
  }

  const int n_chunks = (kv_end - it.kv_begin + CHUNK - 1) / CHUNK;
  // Page id of chunk c: a chunk is 16 keys from a multiple of 16 (partitions
  // start at multiples of the split), so one page, the same for the whole
  // wave: a scalar load, which waits on its own counter instead of behind
  // the data loads in flight (any in-range page past the last chunk).
  auto page_of = [&](int c) -> int32_t {
    return pt[min(it.kv_begin + CHUNK * c, kv_end - 1) >> 4];
  };
  // The 16-byte loads of chunk c (a key past the partition reads the
  // partition's last key instead; such keys are zeroed before use, by
  // zero_tail).
  auto load = [&](uint32_t (&kw)[2][W], uint32_t (&vw)[2][W], int c, int64_t page) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(it.kv_begin + CHUNK * c + 8 * i + ks, kv_end - 1);
      const int64_t off = (page * 16 + (key & 15)) * slot_stride + head_off;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint4 a = *reinterpret_cast<const uint4*>(kp + off + 8 * u);
        const uint4 b = *reinterpret_cast<const uint4*>(vp + off + 8 * u);
        kw[i][4 * u] = a.x; kw[i][4 * u + 1] = a.y; kw[i][4 * u + 2] = a.z; kw[i][4 * u + 3] = a.w;
        vw[i][4 * u] = b.x; vw[i][4 * u + 1] = b.y; vw[i][4 * u + 2] = b.z; vw[i][4 * u + 3] = b.w;
      }
    }
  };
  // Keys of chunk c past the partition hold zeros (only the last chunk can
  // reach past it: a uniform test).
  auto zero_tail = [&](uint32_t (&kw)[2][W], uint32_t (&vw)[2][W], int c) {
    if (it.kv_begin + CHUNK * (c + 1) <= kv_end) return;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool live = it.kv_begin + CHUNK * c + 8 * i + ks < kv_end;
#pragma unroll
      for (int u = 0; u < W; ++u) {
        kw[i][u] = live ? kw[i][u] : 0u;
        vw[i][u] = live ? vw[i][u] : 0u;
      }
    }
  };
  auto compute = [&](uint32_t (&kw)[2][W], uint32_t (&vw)[2][W], int c) {
    zero_tail(kw, vw, c);
    float s[2][G];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool live = it.kv_begin + CHUNK * c + 8 * i + ks < kv_end;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < W; ++u)
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[j][u]),
                                                __builtin_bit_cast(bf16x2_t, kw[i][u]), acc,
                                                false);
        acc = dpp_sum8(acc);
        s[i][j] = live ? acc * scale_log2 : kNegInf;
      }
    }
    bool any_raise = false;
    float alpha[G];
    uint32_t pp[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mt = fmaxf(s[0][j], s[1][j]);
      const bool raise = mt > m[j] + kLazyMax;
      const float m_new = raise ? mt : m[j];
      alpha[j] = raise ? fast_exp2(m[j] - m_new) : 1.0f;
      any_raise |= raise;
      const float msub = (m_new == kNegInf) ? 0.0f : m_new;
      const float p0 = fast_exp2(s[0][j] - msub);
      const float p1 = fast_exp2(s[1][j] - msub);
      l[j] = l[j] * alpha[j] + p0;
      l[j] = l[j] + p1;
      m[j] = m_new;
      pp[j] = pack_bf16x2(p0, p1);
    }
    if (__any(any_raise)) {  // lanes whose heads did not raise have alpha == 1
#pragma unroll
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[j][i] *= alpha[j];
      }
    }
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const uint32_t v_even = __builtin_amdgcn_perm(vw[1][u], vw[0][u], 0x05040100u);
      const uint32_t v_odd = __builtin_amdgcn_perm(vw[1][u], vw[0][u], 0x07060302u);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        o[j][2 * u] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp[j]),
                                                      __builtin_bit_cast(bf16x2_t, v_even),
                                                      o[j][2 * u], false);
        o[j][2 * u + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp[j]),
                                                          __builtin_bit_cast(bf16x2_t, v_odd),
                                                          o[j][2 * u + 1], false);
      }
    }
  };

  // This wave's chunks are wave, wave + 4, ... in that order. NB register
  // buffers rotate: while chunk c is computed, the loads of the next NB - 1
  // chunks are in flight, and page ids run one chunk ahead of the loads that
  // use them. The order of the arithmetic does not depend on NB.
  constexpr int NB = kDecodeBuffers<G>;
  uint32_t kbuf[NB][2][W], vbuf[NB][2][W];
  // Every step issues its chunk's loads, also for a chunk past the partition
  // (those read its last key, in range and never used): with the same loads
  // on every path the compiler's waits for chunk c leave the loads of the
  // chunks after it in flight.
#pragma unroll
  for (int k = 0; k + 1 < NB; ++k) {
    const int cl = wave + 4 * k;
    load(kbuf[k], vbuf[k], cl, page_of(cl));
  }
  int32_t page_next = page_of(wave + 4 * (NB - 1));
  for (int c = wave; c < n_chunks; c += 4 * NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int cc = c + 4 * k;
      if (cc >= n_chunks) break;  // uniform over the wave
      const int cl = cc + 4 * (NB - 1);
      load(kbuf[(k + NB - 1) % NB], vbuf[(k + NB - 1) % NB], cl, page_next);
      page_next = page_of(cl + 4);
      compute(kbuf[k], vbuf[k], cc);
    }
  }

  // ---- combine the 8 key groups of the wave (butterfly over lane ^ 8, 16, 32) ----
  // lane ^ 8: DPP row_ror:8 brings the partner's value. lane ^ 16 and ^ 32:
  // v_permlane16/32_swap return {own value, partner's value} in an order
  // that depends on the lane; combine_sym is symmetric, so both lanes of a
  // pair combine the same two states and get the same bits either way.
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float o2[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) o2[i] = dpp_ror8(o[j][i]);
    combine_sym<DPL>(m[j], l[j], o[j], dpp_ror8(m[j]), dpp_ror8(l[j]), o2);
  }
#pragma unroll
  for (int step = 0; step < 2; ++step) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float oa[DPL], ob[DPL], ma, mb, la, lb;
#pragma unroll
      for (int i = 0; i < DPL; ++i) lane_swap(step, o[j][i], oa[i], ob[i]);
      lane_swap(step, m[j], ma, mb);
      lane_swap(step, l[j], la, lb);
      combine_sym<DPL>(ma, la, oa, mb, lb, ob);
      m[j] = ma;
      l[j] = la;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[j][i] = oa[i];
    }
  }
  if (ks == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int i = 0; i < DPL; ++i) sm_o[wave][j][part * DPL + i] = o[j][i];
      if (part == 0) {
        sm_ml[wave][j][0] = m[j];
        sm_ml[wave][j][1] = l[j];
      }
    }
  }
  __syncthreads();

  // ---- combine the 4 waves in order, normalise, write ----
  for (int e = tid; e < G * D; e += kThreads) {
    const int j = e / D;
    const int d = e % D;
    float mm = sm_ml[0][j][0], ll = sm_ml[0][j][1];
    float oo[1] = {sm_o[0][j][d]};
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float o2[1] = {sm_o[w][j][d]};
      combine_sym<1>(mm, ll, oo, sm_ml[w][j][0], sm_ml[w][j][1], o2);
    }
    float lse_nat = kNegInf;
    float val = 0.0f;
    if (ll > 0.0f) {
      val = oo[0] * (1.0f / ll);
      lse_nat = (mm + fast_log2(ll)) * kLn2;
    }
    const int h = it.kv_head * G + j;
    if (it.state < 0) {
      out[(static_cast<int64_t>(it.q_row0) * num_qo_heads + h) * D + d] = to_bf16_bits(val);
      if (lse_out != nullptr && d == 0)
        lse_out[static_cast<int64_t>(it.q_row0) * num_qo_heads + h] = lse_nat;
    } else {
      const int64_t st = static_cast<int64_t>(it.state) + j;
      o_part[st * D + d] = val;
      if (d == 0) lse_part[st] = lse_nat;
    }
  }
}

// ---------------------------------------------------------------------------
// Latent (MLA) attention, absorbed form: every q head scores against the one
// cached latent row per token (576 bf16: 512 latent + 64 rope dims) and
// averages its first 512 dims (the pages name this MLA path as the one with
// no deterministic mode, sglang PR #43612, commit message and Summary).
//
// One workgroup = one WorkItem = 128 q rows (128 / hb tokens x hb heads of
// one head block, hb = min(Hq, 128); the plan's "kv head" is the head block)
// over one split-KV partition; 8 waves x 16 rows, two waves per SIMD, so one
// wave's softmax, waits and DMA issue overlap the other's MFMAs, and each K/V
// tile staged in LDS serves 128 rows (at 128 heads, each latent row is read
// once per token). Per 32-key tile:
//   K/V staging: the tile's two pages (16 rows x 1152 bytes each, contiguous
//   in the pool) are copied to LDS by DMA, 18 instructions of 1 KB per page
//   spread over the waves. LDS rows are unpadded; the 16-byte chunk c of
//   page row r sits at slot c ^ f(r) (mla_swz), which permutes chunks inside
//   aligned groups of 8 and keeps the K-operand reads (16 rows, one chunk)
//   and the transposing V reads on distinct banks. Four buffers (147 KB,
//   one workgroup per CU): the DMAs of tiles j+1 .. j+3 are in flight while
//   tile j computes, and a wave waits only for its own DMAs of tile j
//   (counted waits). Keys past
//   the partition's end read a valid key of the same page instead; their
//   scores are masked, so they add exact zeros. Page ids come from an LDS
//   copy of the item's page list made once per item.
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys as M, the wave's 16 rows
//   as N, 576 dims as 18 k-steps; layout checked on the GPU with an exact
//   integer probe: A[m][k]: m = l % 16, k = 8 (l / 16) + e; B[k][n]:
//   n = l % 16, same k; D[m][n]: n = l % 16, m = 4 (l / 16) + v), so row n's
//   32 scores sit in lanes n, n + 16, n + 32, n + 48;
//   online softmax per row (lazy max, exp2 with the scale folded in, fp32
//   row sum), max and sums combined over the four lanes with symmetric
//   permlane swaps;
//   O^T += V^T P^T over the wave's 16 rows and all 512 value dims (32 MFMAs):
//   the probabilities stay in registers as the B operand, in the key order
//   the score MFMA left them (slot 8 g + e is key 4 g + e for e < 4 and
//   16 + 4 g + e - 4 otherwise), and V^T is read in that order with
//   ds_read_b64_tr_b16.
// The same invariance rules hold as for the other kernels: tiles anchored at
// the partition start, masked tiles exact no-ops, per-row arithmetic
// independent of the tile holding the row.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kMlaDk = BIA_MLA_QK_DIM;
constexpr int kMlaDv = BIA_MLA_V_DIM;
constexpr int kMlaKeys = 32;                            // keys per tile
constexpr int kMlaRowBytes = kMlaDk * 2;                // 1152, unpadded
constexpr int kMlaPageBytes = 16 * kMlaRowBytes;        // 18432: one page
constexpr int kMlaTileBytes = 2 * kMlaPageBytes;        // 36864
constexpr int kMlaBufs = 4;
constexpr int kMlaPageDma = kMlaPageBytes / 1024;       // 18 DMA instructions per page
constexpr int kMlaWaves = 8;                            // two per SIMD
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kMlaDmaPerWave = (kMlaPageDma + kMlaWaves - 1) / kMlaWaves;  // i = wave + 8 k
constexpr int kMlaMaxPages = BIA_MLA_MAX_SPLIT / 16;    // page list held in LDS
static_assert(kMlaPageBytes % 1024 == 0, "a page is whole DMA instructions");

// max and sum over the lanes n, n ^ 16, n ^ 32, n ^ 48 (symmetric: every lane
// of the four gets the same bits)
__device__ __forceinline__ float quad_max(float x) {
  float a, b;
  lane_swap(0, x, a, b);
  x = fmaxf(a, b);
  lane_swap(1, x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float quad_sum(float x) {
  float a, b;
  lane_swap(0, x, a, b);
  x = a + b;
  lane_swap(1, x, a, b);
  return a + b;
}

// Chunk permutation of page row r (0..15): chunk c sits at slot c ^ f(r),
// f(r) = r % 8. Chosen by timing the two read patterns on gfx950 (eight
// waves per CU reading at fixed per-lane offsets): the K reads (b128, 16
// rows x one chunk) and the transposing V^T reads (rows 0..7 or 8..15, two
// adjacent chunks) both run at the conflict-free rate with r % 8;
// (r / 2) % 8 made the V^T reads 7 % slower and 2 ((r / 2) % 4) + r / 8
// made the K reads 40 % slower. A row is 1152 bytes, so no swizzle leaves
// every row on the same banks.
__device__ __forceinline__ int mla_swz(int r) { return r & 7; }
// Slot of 16-byte chunk c in page row r (an involution).
__device__ __forceinline__ int mla_slot(int r, int c) { return c ^ mla_swz(r); }

// Wait until at most n of this wave's DMAs are outstanding (n a multiple of
// the per-tile count; vmcnt counts in issue order).
__device__ __forceinline__ void mla_wait(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
  }
}

__global__ void __launch_bounds__(kMlaThreads, 1)
mla_kernel(const WorkItem* __restrict__ items, const uint16_t* __restrict__ q,
           const uint16_t* __restrict__ kvp, const int32_t* __restrict__ page_table,
           float scale_log2, int num_qo_heads, int hb_shift, int split,
           uint16_t* __restrict__ out, float* __restrict__ lse_out,
           float* __restrict__ o_part, float* __restrict__ lse_part) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kMlaBufs * kMlaTileBytes];
  __shared__ int32_t lds_pages[kMlaMaxPages];
  const WorkItem it = items[blockIdx.x];
  if (it.n_tok == 0) return;  // padding of the XCD-interleaved launch order
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;   // 16-lane group
  const int n16 = lane & 15;  // the lane's row among the wave's 16 (and its M index)
  const int hb = 1 << hb_shift;
  const int x = wave * 16 + n16;  // row of the 128-row tile
  const int tok = x >> hb_shift;
  const int hq = it.kv_head * hb + (x & (hb - 1));
  const bool row_valid = tok < it.n_tok;
  const int pos = row_valid ? it.pos0 + tok : -1;
  const int wave_pos0 = it.pos0 + ((wave * 16) >> hb_shift);
  const int64_t row_idx = static_cast<int64_t>(it.q_row0 + tok) * num_qo_heads + hq;

  // Q^T fragments (B operand): row n16, dims 32 s + 8 g4 .. + 7
  bf16x8 qf[kMlaDk / 32];
#pragma unroll
  for (int s = 0; s < kMlaDk / 32; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row_valid)
      w = *reinterpret_cast<const uint4*>(q + row_idx * kMlaDk + 32 * s + 8 * g4);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }

  const int last = it.pos0 + it.n_tok - 1;
  const int kv_end = min(it.kv_begin + split, last + 1);
  const int n_tiles = (kv_end - it.kv_begin + kMlaKeys - 1) / kMlaKeys;
  const int first_page = it.kv_begin >> 4;
  const int n_pages = ((kv_end - 1) >> 4) - first_page + 1;  // <= kMlaMaxPages (plan check)
  const int32_t* pt = page_table + it.page_off + first_page;
  for (int i = tid; i < n_pages; i += kMlaThreads) lds_pages[i] = pt[i];
  // Q and the page list are waited for here, before any DMA is in flight:
  // the DMAs are inline asm the compiler does not count, and a later
  // compiler wait for these loads would also wait for the DMAs.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // Register placement (two waves per SIMD, 256 registers each): Q^T, O
  // and everything else in VGPRs, none in AGPRs. With the library built for
  // VGPR-form MFMAs the tile loop moves nothing between the two register
  // files (an even VGPR/AGPR split at this occupancy spilled, and at one wave
  // per SIMD the allocator copied the 128 O registers between the files
  // around the PV MFMAs of every tile).
#pragma unroll
  for (int s = 0; s < kMlaDk / 32; ++s) asm volatile("" : "+v"(qf[s]));
  __syncthreads();

  // DMA of tile t into buffer t % 4: instruction i (0..17) of page half ph
  // copies LDS bytes ph * 18432 + 1024 i + 16 lane .. + 15 of the tile, which
  // hold tile row r = 16 ph + (1024 i + 16 lane) / 1152 at slot
  // ((1024 i + 16 lane) % 1152) / 16 = mla_slot(r, c) for chunk c. Wave w
  // issues i = w, w + 8, ..: 6 instructions per tile for waves 0-1, 4 for
  // waves 2-7 (the same count for every tile, ragged ones included).
  const uint32_t lds_base = lds_offset(lds);
  uint32_t dma_off[kMlaDmaPerWave];  // byte offset of this lane's chunk in its page
  int dma_row[kMlaDmaPerWave];       // its row in the page
#pragma unroll
  for (int k = 0; k < kMlaDmaPerWave; ++k) {
    const int i = wave + kMlaWaves * k;
    const int p = 1024 * i + 16 * lane;
    const int rr = p / kMlaRowBytes;
    const int c = mla_slot(rr, (p % kMlaRowBytes) / 16);  // the slot map is an involution
    dma_row[k] = rr;
    dma_off[k] = static_cast<uint32_t>(rr * kMlaRowBytes + c * 16);
  }
  const int dma_count = 2 * ((kMlaPageDma - wave + kMlaWaves - 1) / kMlaWaves);  // 6 or 4
  auto issue = [&](int t) {
    const int t0 = it.kv_begin + kMlaKeys * t;
    const bool ragged = t0 + kMlaKeys > kv_end;
    const int last_slot = (kv_end - 1) & 15;
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int pi = min(2 * t + ph, n_pages - 1);
      const int32_t page = __builtin_amdgcn_readfirstlane(lds_pages[pi]);
      const uint16_t* pbase = kvp + static_cast<int64_t>(page) * 16 * kMlaDk;
      const uint32_t buf_lds = lds_base + (t % kMlaBufs) * kMlaTileBytes + ph * kMlaPageBytes;
#pragma unroll
      for (int k = 0; k < kMlaDmaPerWave; ++k) {
        const int i = wave + kMlaWaves * k;
        if (i < kMlaPageDma) {  // wave-uniform
          uint32_t off = dma_off[k];
          if (ragged && t0 + 16 * ph + dma_row[k] >= kv_end)  // past the keys: a valid key's chunk
            off = static_cast<uint32_t>(last_slot * kMlaRowBytes) + off % kMlaRowBytes;
          lds_dma16_sbase(off, pbase, buf_lds + 1024 * i);
        }
      }
    }
  };

  float m = kNegInf;   // running max (base-2 scaled), stale by < kLazyMax
  float lsum = 0.0f;   // this lane's share of the row's running sum
  f32x4 o[kMlaDv / 16];
#pragma unroll
  for (int b = 0; b < kMlaDv / 16; ++b) o[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // K operand of k-step s, key block kb: tile row 16 kb + n16 (f depends on
  // n16 only), chunk 4 s + g4 -> slot 8 (s / 2) + ((4 (s % 2) + g4) ^ f).
  const int fk = mla_swz(n16);
  const int k_off[2] = {n16 * kMlaRowBytes + 16 * ((0 + g4) ^ fk),
                        n16 * kMlaRowBytes + 16 * ((4 + g4) ^ fk)};
  // V^T operand of dim block b: rows 4 g4 + n16 / 4 (+ 16), dims 16 b + 4 (n16 % 4):
  // chunk 2 b + h (h = (n16 % 4) / 2), byte (n16 % 2) * 8 in it -> slot
  // 8 (b / 4) + ((2 (b % 4) + h) ^ f).
  const int vr = 4 * g4 + (n16 >> 2);
  const int fv = mla_swz(vr);
  const int vh = (n16 & 3) >> 1;
  int v_off[4];
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4)
    v_off[b4] = vr * kMlaRowBytes + 16 * ((2 * b4 + vh) ^ fv) + 8 * (n16 & 1);

  // A wave whose rows are all past the item's tokens (decode with fewer than
  // 128 rows, a request's last tile) skips the MFMAs; it still issues its DMAs
  // and meets every barrier.
  const bool wave_active = ((wave * 16) >> hb_shift) < it.n_tok;
  auto compute = [&](int j, int buf) {
    if (!wave_active) return;
    const uint8_t* base = &lds[buf * kMlaTileBytes];
    // ---- scores: S^T for keys 16 kb + m (m = n16) x the wave's 16 rows ----
    // MFMA i = 2 s + kb; its K fragment is read kAhead MFMAs earlier (ring of
    // kRing registers), each slot fenced so the reads stay ahead.
    constexpr int kAhead = 3, kRing = 4, kNs = 2 * (kMlaDk / 32);
    auto kfrag = [&](int i) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                            base + (i & 1) * kMlaPageBytes +
                                            k_off[(i >> 1) & 1] + 128 * (i >> 2)));
    };
    f32x4 sc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
    bf16x8 kf[kRing];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kf[i] = kfrag(i);
#pragma unroll
    for (int i = 0; i < kNs; ++i) {
      sc[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[i % kRing], qf[i >> 1], sc[i & 1],
                                                          0, 0, 0);
      if (i + kAhead < kNs) kf[(i + kAhead) % kRing] = kfrag(i + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first V^T fragments go out before the softmax (they do not need P)
    auto vfrag = [&](int b) -> bf16x8 {
      const uint8_t* vb = base + v_off[b & 3] + 128 * (b >> 2);
      const uint2 lo = lds_read_tr16(vb);
      const uint2 hi = lds_read_tr16(vb + kMlaPageBytes);
      return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    bf16x8 vf[kRing];
#pragma unroll
    for (int b = 0; b < kAhead; ++b) vf[b] = vfrag(b);
    const int t0 = it.kv_begin + kMlaKeys * j;
    if (t0 + kMlaKeys - 1 > wave_pos0) {  // wave-uniform: some key is past some row
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sc[kb][v] = (t0 + 16 * kb + 4 * g4 + v <= pos) ? sc[kb][v] : kNegInf;
    }
    // ---- online softmax of the row ----
    float mx = sc[0][0];
#pragma unroll
    for (int v = 1; v < 4; ++v) mx = fmaxf(mx, sc[0][v]);
#pragma unroll
    for (int v = 0; v < 4; ++v) mx = fmaxf(mx, sc[1][v]);
    const float mt = quad_max(mx) * scale_log2;
    const bool raise = mt > m + kLazyMax;  // true on the first tile with a visible key
    const float m_new = raise ? mt : m;
    const float alpha = raise ? fast_exp2(m - m_new) : 1.0f;
    const float neg_m = (m_new == kNegInf) ? 0.0f : -m_new;
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[kb][v] = fast_exp2(__builtin_fmaf(sc[kb][v], scale_log2, neg_m));
        psum += p[kb][v];
      }
    const uint4 pw = make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3]));
    if (__any(raise)) {  // lanes that did not raise have alpha == 1 exactly
      lsum *= alpha;
#pragma unroll
      for (int b = 0; b < kMlaDv / 16; ++b) o[b] *= alpha;
    }
    lsum += psum;
    m = m_new;
    // ---- O^T += V^T P^T: 32 blocks of 16 value dims, reads kAhead ahead ----
#pragma unroll
    for (int b = 0; b < kMlaDv / 16; ++b) {
      o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[b % kRing], __builtin_bit_cast(bf16x8, pw),
                                                     o[b], 0, 0, 0);
      if (b + kAhead < kMlaDv / 16) vf[(b + kAhead) % kRing] = vfrag(b + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < kMlaDv / 16; ++b) asm volatile("" : "+v"(o[b]));  // O stays in VGPRs
  };

  // DMAs of tiles 0 .. 2 ahead of the loop; tile j+3 goes into the buffer of
  // tile j-1 once every wave has passed the barrier that follows tile j-1.
  for (int t = 0; t < min(n_tiles, kMlaBufs - 1); ++t) issue(t);
  for (int j = 0; j < n_tiles; ++j) {
    mla_wait(dma_count * min(kMlaBufs - 2, n_tiles - 1 - j));  // this wave's tile-j DMAs done
    __syncthreads();  // every wave's are; every wave is done with tile j-1
    if (j + kMlaBufs - 1 < n_tiles) issue(j + kMlaBufs - 1);
    compute(j, j % kMlaBufs);
  }

  // ---- this partition's state for the row: o = O / l, lse = m + log l ----
  const float l_row = quad_sum(lsum);
  if (!row_valid) return;
  float lse_nat = kNegInf;
  float inv = 0.0f;
  if (l_row > 0.0f) {
    inv = 1.0f / l_row;
    lse_nat = (m + fast_log2(l_row)) * kLn2;
  }
  if (it.state < 0) {
    uint16_t* orow = out + row_idx * kMlaDv;
#pragma unroll
    for (int b = 0; b < kMlaDv / 16; ++b) {
      *reinterpret_cast<uint2*>(orow + 16 * b + 4 * g4) =
          make_uint2(pack_bf16x2(o[b][0] * inv, o[b][1] * inv),
                     pack_bf16x2(o[b][2] * inv, o[b][3] * inv));
    }
    if (lse_out != nullptr && g4 == 0) lse_out[row_idx] = lse_nat;
  } else {
    const int64_t st = static_cast<int64_t>(it.state) + x;
    float* orow = o_part + st * kMlaDv;
#pragma unroll
    for (int b = 0; b < kMlaDv / 16; ++b)
      *reinterpret_cast<float4*>(orow + 16 * b + 4 * g4) =
          make_float4(o[b][0] * inv, o[b][1] * inv, o[b][2] * inv, o[b][3] * inv);
    if (g4 == 0) lse_part[st] = lse_nat;
  }
}

// ---------------------------------------------------------------------------
// Latent (MLA) decode with at most 16 q heads: one wave per work item (the
// item's q heads are rows 0 .. Hq - 1 of the wave's 16), kMlaDecWaves (3)
// consecutive items per workgroup (measured faster than spreading the items
// over at least one workgroup per CU), no workgroup barrier. Each wave streams its partition in
// 16-key tiles (one page each) through two LDS buffers of its own (DMA,
// counted waits, the same swizzled unpadded rows as mla_kernel):
//   S^T = K Q^T: 18 v_mfma_f32_16x16x32_bf16 (keys as M, rows as N);
//   online softmax per row over the four lanes that hold it;
//   O^T += V^T P^T: 32 v_mfma_f32_16x16x16_bf16, one per 16 value dims. The
//   16x16x16 B operand (k = 4 (l / 16) + e) is exactly the score MFMA's
//   output layout, so P goes in as the scores left it, and V^T is one
//   transposing read per MFMA.
// Rows past the partition's end read a valid key of the same page; their
// scores are masked. Per-row arithmetic depends only on the item, so decode
// stays batch-invariant (it differs from prefill's 32-key tiles).
// ---------------------------------------------------------------------------
constexpr int kMlaDecTileKeys = 16;
constexpr int kMlaDecMaxPages = 128;  // page list per wave: splits up to 2048 keys
typedef short v4i16_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void mla_dec_wait(bool next_in_flight) {
  if (next_in_flight) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Items (one wave each) per workgroup; one workgroup per CU (LDS). Three
// spread the B = 64, 16-head decode's items over more CUs than four in one
// round (0.278-0.282 against 0.284-0.286 ms on one box); two need a second
// round (0.331 ms).
constexpr int kMlaDecWaves = 3;

__global__ void __launch_bounds__(64 * kMlaDecWaves, 1)
mla_decode_kernel(const WorkItem* __restrict__ items, int n_items,
                  const uint16_t* __restrict__ q, const uint16_t* __restrict__ kvp,
                  const int32_t* __restrict__ page_table, float scale_log2, int num_qo_heads,
                  int hb, int split, uint16_t* __restrict__ out, float* __restrict__ lse_out,
                  float* __restrict__ o_part, float* __restrict__ lse_part) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kMlaDecWaves][2][kMlaPageBytes];
  __shared__ int32_t lds_pages[kMlaDecWaves][kMlaDecMaxPages];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * kMlaDecWaves + wave;
  if (item >= n_items) return;  // no barrier below: waves are independent
  const WorkItem it = items[item];
  if (it.n_tok == 0) return;
  const int g4 = lane >> 4;
  const int n16 = lane & 15;  // row: q head kv_head * hb + n16 when n16 < hb
  const bool row_valid = n16 < hb;
  const int pos = row_valid ? it.pos0 : -1;
  const int64_t row_idx =
      static_cast<int64_t>(it.q_row0) * num_qo_heads + it.kv_head * hb + n16;

  bf16x8 qf[kMlaDk / 32];
#pragma unroll
  for (int s = 0; s < kMlaDk / 32; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row_valid)
      w = *reinterpret_cast<const uint4*>(q + row_idx * kMlaDk + 32 * s + 8 * g4);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }
  const int kv_end = min(it.kv_begin + split, it.pos0 + 1);
  const int n_tiles = (kv_end - it.kv_begin + kMlaDecTileKeys - 1) / kMlaDecTileKeys;
  const int32_t* pt = page_table + it.page_off + (it.kv_begin >> 4);
  int32_t* my_pages = lds_pages[wave];
  for (int i = lane; i < n_tiles; i += 64) my_pages[i] = pt[i];  // one page per tile
  // Q and the page ids are waited for before any DMA is in flight.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  // Q^T fragments in AGPRs, O in VGPRs, as in mla_kernel.
#pragma unroll
  for (int s = 0; s < kMlaDk / 32; ++s) asm volatile("" : "+a"(qf[s]));

  // DMA of tile t: 18 instructions of 1 KB; instruction i, lane l copies LDS
  // bytes 1024 i + 16 l (row rr, slot sl) from chunk sl ^ f(rr) of row rr.
  const uint32_t lds_base = lds_offset(&lds[wave][0][0]);
  const int last_slot = (kv_end - 1) & 15;
  auto issue = [&](int t) {
    const int32_t page = __builtin_amdgcn_readfirstlane(my_pages[t]);
    const uint16_t* pbase = kvp + static_cast<int64_t>(page) * 16 * kMlaDk;
    const int t0 = it.kv_begin + kMlaDecTileKeys * t;
    const int valid_rows = kv_end - t0;  // >= 1
    const uint32_t buf = lds_base + (t & 1) * kMlaPageBytes;
#pragma unroll
    for (int i = 0; i < kMlaPageDma; ++i) {
      const int p = 1024 * i + 16 * lane;
      int rr = p / kMlaRowBytes;
      const int c = mla_slot(rr, (p % kMlaRowBytes) / 16);
      if (rr >= valid_rows) rr = last_slot;  // past the keys: a valid key of this page
      lds_dma16_sbase(static_cast<uint32_t>(rr * kMlaRowBytes + c * 16), pbase, buf + 1024 * i);
    }
  };

  const int fk = mla_swz(n16);
  const int k_off[2] = {n16 * kMlaRowBytes + 16 * ((0 + g4) ^ fk),
                        n16 * kMlaRowBytes + 16 * ((4 + g4) ^ fk)};
  // V^T of dim block b: rows 4 g4 + n16 / 4 (the 4 keys of this lane group),
  // dims 16 b + 4 (n16 % 4) .. + 3
  const int vr = 4 * g4 + (n16 >> 2);
  const int fv = mla_swz(vr);
  const int vh = (n16 & 3) >> 1;
  int v_off[4];
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4)
    v_off[b4] = vr * kMlaRowBytes + 16 * ((2 * b4 + vh) ^ fv) + 8 * (n16 & 1);

  float m = kNegInf;
  float lsum = 0.0f;
  f32x4 o[kMlaDv / 16];
#pragma unroll
  for (int b = 0; b < kMlaDv / 16; ++b) o[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int t) {
    const uint8_t* base = &lds[wave][t & 1][0];
    constexpr int kAhead = 6, kRing = 8, kNs = kMlaDk / 32;
    auto kfrag = [&](int s) -> bf16x8 {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(base + k_off[s & 1] + 128 * (s >> 1)));
    };
    f32x4 sc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 kf[kRing];
#pragma unroll
    for (int s = 0; s < kAhead; ++s) kf[s] = kfrag(s);
#pragma unroll
    for (int s = 0; s < kNs; ++s) {
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s % kRing], qf[s], sc, 0, 0, 0);
      if (s + kAhead < kNs) kf[(s + kAhead) % kRing] = kfrag(s + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
    auto vfrag = [&](int b) -> v4i16_t {
      return __builtin_bit_cast(v4i16_t, lds_read_tr16(base + v_off[b & 3] + 128 * (b >> 2)));
    };
    v4i16_t vf[kRing];
#pragma unroll
    for (int b = 0; b < kAhead; ++b) vf[b] = vfrag(b);
    const int t0 = it.kv_begin + kMlaDecTileKeys * t;
    if (t0 + kMlaDecTileKeys - 1 > it.pos0) {  // a key past the row (decode: the last tile)
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = (t0 + 4 * g4 + v <= pos) ? sc[v] : kNegInf;
    }
    if (!row_valid) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = kNegInf;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    const float mt = quad_max(mx) * scale_log2;
    const bool raise = mt > m + kLazyMax;
    const float m_new = raise ? mt : m;
    const float alpha = raise ? fast_exp2(m - m_new) : 1.0f;
    const float neg_m = (m_new == kNegInf) ? 0.0f : -m_new;
    float p[4];
    float psum = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = fast_exp2(__builtin_fmaf(sc[v], scale_log2, neg_m));
      psum += p[v];
    }
    const v4i16_t pw = __builtin_bit_cast(
        v4i16_t, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
    if (__any(raise)) {
      lsum *= alpha;
#pragma unroll
      for (int b = 0; b < kMlaDv / 16; ++b) o[b] *= alpha;
    }
    lsum += psum;
    m = m_new;
#pragma unroll
    for (int b = 0; b < kMlaDv / 16; ++b) {
      o[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[b % kRing], pw, o[b], 0, 0, 0);
      if (b + kAhead < kMlaDv / 16) vf[(b + kAhead) % kRing] = vfrag(b + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < kMlaDv / 16; ++b) asm volatile("" : "+v"(o[b]));
  };

  issue(0);
  if (n_tiles > 1) issue(1);
  for (int t = 0; t < n_tiles; ++t) {
    mla_dec_wait(t + 1 < n_tiles);  // this tile's DMAs have landed
    compute(t);                     // its LDS reads are all complete when it returns
    if (t + 2 < n_tiles) issue(t + 2);
  }

  const float l_row = quad_sum(lsum);
  if (!row_valid) return;
  float lse_nat = kNegInf;
  float inv = 0.0f;
  if (l_row > 0.0f) {
    inv = 1.0f / l_row;
    lse_nat = (m + fast_log2(l_row)) * kLn2;
  }
  if (it.state < 0) {
    uint16_t* orow = out + row_idx * kMlaDv;
#pragma unroll
    for (int b = 0; b < kMlaDv / 16; ++b)
      *reinterpret_cast<uint2*>(orow + 16 * b + 4 * g4) =
          make_uint2(pack_bf16x2(o[b][0] * inv, o[b][1] * inv),
                     pack_bf16x2(o[b][2] * inv, o[b][3] * inv));
    if (lse_out != nullptr && g4 == 0) lse_out[row_idx] = lse_nat;
  } else {
    const int64_t st = static_cast<int64_t>(it.state) + n16;
    float* orow = o_part + st * kMlaDv;
#pragma unroll
    for (int b = 0; b < kMlaDv / 16; ++b)
      *reinterpret_cast<float4*>(orow + 16 * b + 4 * g4) =
          make_float4(o[b][0] * inv, o[b][1] * inv, o[b][2] * inv, o[b][3] * inv);
    if (g4 == 0) lse_part[st] = lse_nat;
  }
}

// ---------------------------------------------------------------------------
// a4 on MFMA: decode (decode_mfma_kernel<D, G>, D = 64 or 128). One workgroup of
// eight waves runs one item (request, kv head, partition); the partition's
// 16-key tiles (one page each) go round-robin to the waves, tile t to wave
// t % 8, and each wave keeps its own online-softmax state. Per tile and wave:
//   K and V rows of the kv head reach the wave's LDS buffers by DMA (D / 32 +
//   D / 32 instructions of 1 KB), NB buffers deep, counted waits;
//   S^T = K Q^T: D / 32 v_mfma_f32_16x16x32_bf16, keys as M, the group's G q
//   heads as N (16 columns, G of them real);
//   online softmax per q head over the lanes n, n + 16, n + 32, n + 48;
//   O^T += V^T P^T: D / 16 v_mfma_f32_16x16x16_bf16, P as the scores left it,
//   V^T by transposing reads.
// The eight waves' states fold in ascending wave order (combine_sym), as in
// decode_kernel. The page list of the partition is copied to LDS once, so the
// tile loop holds no global load the compiler would count.
// ---------------------------------------------------------------------------
// Waves per item: eight keep twice the tiles of a small batch in flight at the
// same waves per CU as two four-wave workgroups (one workgroup per CU: LDS).
constexpr int kDecMfmaWaves = 8;
constexpr int kDecMfmaMaxPages = 1024;  // page list in LDS: splits up to 16384 keys
constexpr int kDecMfmaBufs = 2;         // tile buffers per wave

// Chunk permutation of tile row r: chunk c sits at slot c ^ f(r).
// D = 128 (16 chunks of 16 bytes, a row per 256-byte bank cycle): f(r) =
// 2 (r % 8) + r / 8. The K reads (row n16, one chunk, 16 rows per 16 lanes)
// then take 16 distinct slots of the cycle, and the transposing V reads (rows
// 4 g4 .. 4 g4 + 3, 32 bytes each, and any 8 consecutive rows) take distinct
// 32-byte pairs of it.
// D = 64 (8 chunks, two rows per cycle, rows of one parity share its banks):
// f(r) = 2 ((r / 2) % 4) + r / 8, distinct over the 8 rows of each parity
// (K reads), and its pair index (r / 2) % 4 distinct over the rows of equal
// parity in any 4 or 8 consecutive rows (V reads).
template <int D>
__device__ __forceinline__ int dec_swz(int r) {
  if constexpr (D == 128) return ((r & 7) << 1) | (r >> 3);
  else return (((r >> 1) & 3) << 1) | (r >> 3);
}

template <int N>
__device__ __forceinline__ void dec_wait(int tiles_ahead) {
  // N DMA instructions per tile; tiles_ahead (0 .. 2) tiles may stay in flight
  if (tiles_ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * N) : "memory");
  else if (tiles_ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D, int G>
// (a register budget of 128 VGPRs: the kernel takes 103 at D = 128)
__global__ void __launch_bounds__(64 * kDecMfmaWaves, 2)
decode_mfma_kernel(const WorkItem* __restrict__ items, const uint16_t* __restrict__ q,
                   const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                   const int32_t* __restrict__ page_table, float scale_log2, int num_qo_heads,
                   int num_kv_heads, int split, uint16_t* __restrict__ out,
                   float* __restrict__ lse_out, float* __restrict__ o_part,
                   float* __restrict__ lse_part) {
  constexpr int RB = 2 * D;        // bytes of one key row of one head
  constexpr int TB = 16 * RB;      // one tensor's tile: 16 keys
  constexpr int NI = TB / 1024;    // DMA instructions per tensor tile
  constexpr int RPI = 1024 / RB;   // rows per DMA instruction (4 or 8)
  constexpr int CPR = RB / 16;     // 16-byte chunks per row (16 or 8)
  constexpr int NS = D / 32;       // score k-steps
  constexpr int NV = D / 16;       // PV dim blocks
  constexpr int NB = kDecMfmaBufs;
  static_assert(kDecMfmaWaves * NB * 2 * TB >= kDecMfmaWaves * (G * D + 2 * G) * 4,
                "the wave states fit in the tile buffers");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kDecMfmaWaves][NB][2 * TB];
  __shared__ int32_t lds_pages[kDecMfmaMaxPages];

  const WorkItem it = items[blockIdx.x];
  if (it.n_tok == 0) return;  // a fixed-capacity slot past the request's partitions
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;
  const int n16 = lane & 15;       // q head kv_head * G + n16 when n16 < G
  const bool row_valid = n16 < G;

  const int kv_end = min(it.kv_begin + split, it.kv_len);
  const int n_tiles = (kv_end - it.kv_begin + 15) >> 4;
  const int32_t* pt = page_table + it.page_off + (it.kv_begin >> 4);
  for (int i = tid; i < n_tiles; i += 64 * kDecMfmaWaves) lds_pages[i] = pt[i];

  // Q^T fragments (B operand): q head n16, dims 32 s + 8 g4 .. + 7; zero for
  // the columns past the group
  const int64_t q_row = static_cast<int64_t>(it.q_row0) * num_qo_heads + it.kv_head * G +
                        (row_valid ? n16 : 0);
  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row_valid) w = *reinterpret_cast<const uint4*>(q + q_row * D + 32 * s + 8 * g4);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }
  // q and the page list are waited for before any DMA is in flight
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();

  // DMA of tile t into buffer b: tensor x, instruction i fills rows RPI i ..
  // RPI i + RPI - 1 of the buffer's x half; lane l puts 16 bytes in slot
  // l % CPR of row RPI i + l / CPR, i.e. chunk (l % CPR) ^ f(row). Keys
  // past the partition read its last key (same page: tiles are page-aligned).
  const uint32_t lds_base = lds_offset(&lds[wave][0][0]);
  const int64_t slot_bytes = static_cast<int64_t>(num_kv_heads) * RB;
  const int64_t head_bytes = static_cast<int64_t>(it.kv_head) * RB;
  const int last_key = kv_end - 1;
  auto issue = [&](int t, int b) {
    const int32_t page = __builtin_amdgcn_readfirstlane(lds_pages[t]);
    const int64_t page_bytes = static_cast<int64_t>(page) * 16 * slot_bytes + head_bytes;
    const int t0 = it.kv_begin + 16 * t;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint8_t* base = reinterpret_cast<const uint8_t*>(x == 0 ? kp : vp) + page_bytes;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = RPI * i + lane / CPR;
        const int key = min(t0 + r, last_key);
        const uint32_t off =
            static_cast<uint32_t>((key & 15) * slot_bytes + 16 * ((lane % CPR) ^ dec_swz<D>(r)));
        lds_dma16_sbase(off, base, lds_base + b * (2 * TB) + x * TB + 1024 * i);
      }
    }
  };

  // K fragment s (A operand): key n16, dims 32 s + 8 g4 .., chunk 4 s + g4
  const int fk = dec_swz<D>(n16);
  // V^T fragment of dim block b: keys 4 g4 .. 4 g4 + 3 (row vr and the three
  // after it, transposed by the read), dims 16 b + 4 (n16 % 4) .. + 3
  const int vr = 4 * g4 + (n16 >> 2);
  const int fv = dec_swz<D>(vr);

  float m = kNegInf;
  float lsum = 0.0f;
  f32x4 o[NV];
#pragma unroll
  for (int b = 0; b < NV; ++b) o[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int t, int b) {
    const uint8_t* kb = &lds[wave][b][0];
    const uint8_t* vb = kb + TB;
    bf16x8 kf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kf[s] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(kb + n16 * RB + 16 * ((4 * s + g4) ^ fk)));
    v4i16_t vf[NV];
#pragma unroll
    for (int d = 0; d < NV; ++d)
      vf[d] = __builtin_bit_cast(
          v4i16_t, lds_read_tr16(vb + vr * RB + 16 * ((2 * d + ((n16 & 3) >> 1)) ^ fv) +
                                 8 * (n16 & 1)));
    f32x4 sc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < NS; ++s)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], sc, 0, 0, 0);
    // lane (n16, g4) holds keys t0 + 4 g4 .. + 3 of q head n16
    const int t0 = it.kv_begin + 16 * t;
    if (t0 + 16 > kv_end) {  // the partition's last, partly filled tile
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = (t0 + 4 * g4 + v < kv_end) ? sc[v] : kNegInf;
    }
    if (!row_valid) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = kNegInf;
    }
    const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    const float mt = quad_max(mx) * scale_log2;
    const bool raise = mt > m + kLazyMax;
    const float m_new = raise ? mt : m;
    const float alpha = raise ? fast_exp2(m - m_new) : 1.0f;
    const float neg_m = (m_new == kNegInf) ? 0.0f : -m_new;
    float p[4];
    float psum = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = fast_exp2(__builtin_fmaf(sc[v], scale_log2, neg_m));
      psum += p[v];
    }
    const v4i16_t pw = __builtin_bit_cast(
        v4i16_t, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
    if (__any(raise)) {  // lanes whose q head did not raise have alpha == 1
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < NV; ++d) o[d] *= alpha;
    }
    lsum += psum;
    m = m_new;
#pragma unroll
    for (int d = 0; d < NV; ++d)
      o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[d], pw, o[d], 0, 0, 0);
  };

  // this wave's tiles: wave, wave + 4, ...; NB in flight, each sent into the
  // buffer the tile before it has finished with
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + kDecMfmaWaves - 1) / kDecMfmaWaves : 0;
#pragma unroll
  for (int k = 0; k < NB; ++k)
    if (k < my_tiles) issue(wave + kDecMfmaWaves * k, k);
  for (int k = 0; k < my_tiles; ++k) {
    dec_wait<2 * NI>(min(NB - 1, my_tiles - 1 - k));  // tile k has landed
    compute(wave + kDecMfmaWaves * k, k % NB);         // its LDS reads are done on return
    if (k + NB < my_tiles) issue(wave + kDecMfmaWaves * (k + NB), k % NB);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- fold the waves' states in order (their buffers are free now) ----
  const float l_row = quad_sum(lsum);
  __syncthreads();  // every wave is past its last tile
  float* sm_o = reinterpret_cast<float*>(&lds[0][0][0]);  // [wave][G][D]
  float* sm_ml = sm_o + kDecMfmaWaves * G * D;             // [wave][G][2]
  if (row_valid) {
#pragma unroll
    for (int d = 0; d < NV; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) sm_o[(wave * G + n16) * D + 16 * d + 4 * g4 + v] = o[d][v];
    if (g4 == 0) {
      sm_ml[(wave * G + n16) * 2] = m;
      sm_ml[(wave * G + n16) * 2 + 1] = l_row;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 64 * kDecMfmaWaves) {
    const int j = e / D;
    const int d = e % D;
    float mm = sm_ml[j * 2], ll = sm_ml[j * 2 + 1];
    float oo[1] = {sm_o[j * D + d]};
#pragma unroll
    for (int w = 1; w < kDecMfmaWaves; ++w) {
      const float o2[1] = {sm_o[(w * G + j) * D + d]};
      combine_sym<1>(mm, ll, oo, sm_ml[(w * G + j) * 2], sm_ml[(w * G + j) * 2 + 1], o2);
    }
    float lse_nat = kNegInf;
    float val = 0.0f;
    if (ll > 0.0f) {
      val = oo[0] * (1.0f / ll);
      lse_nat = (mm + fast_log2(ll)) * kLn2;
    }
    const int h = it.kv_head * G + j;
    if (it.state < 0) {
      out[(static_cast<int64_t>(it.q_row0) * num_qo_heads + h) * D + d] = to_bf16_bits(val);
      if (lse_out != nullptr && d == 0)
        lse_out[static_cast<int64_t>(it.q_row0) * num_qo_heads + h] = lse_nat;
    } else {
      const int64_t st = static_cast<int64_t>(it.state) + j;
      o_part[st * D + d] = val;
      if (d == 0) lse_part[st] = lse_nat;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of a tile's partitions (prefill rows spanning several partitions,
// decode requests longer than one partition): row x of MergeItem mi folds
// slots state0 + k * stride + x, k ascending, with fold_state. D/4 threads
// per row, 4 dims each.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kThreads)
merge_tiles_kernel(const MergeItem* __restrict__ merges, const float* __restrict__ o_part,
                   const float* __restrict__ lse_part, int num_qo_heads, int group_shift,
                   uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int TPR = D / 4;              // threads per row
  constexpr int RPB = kThreads / TPR;     // rows per workgroup
  const MergeItem mi = merges[blockIdx.x];
  const int g = 1 << group_shift;
  const int rows = mi.n_tok * g;
  const int d0 = (threadIdx.x % TPR) * 4;
  constexpr int kBatch = 8;  // states loaded ahead of their fold
  // workgroup (i, c) takes rows c RPB .. c RPB + RPB - 1 of merge item i, so
  // an item's rows spread over the chip (a 128-head latent decode is one
  // 128-row item per request)
  const int x = blockIdx.y * RPB + threadIdx.x / TPR;
  if (x < rows) {
    float M = kNegInf, sum = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < mi.n_splits; k0 += kBatch) {
      // issue the loads of up to kBatch states, then fold them in order
      float4 v[kBatch];
      float l[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (k0 + i < mi.n_splits) {
          const int64_t st = static_cast<int64_t>(mi.state0) +
                             static_cast<int64_t>(k0 + i) * mi.stride + x;
          v[i] = *reinterpret_cast<const float4*>(o_part + st * D + d0);
          l[i] = lse_part[st];
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (k0 + i < mi.n_splits) {
          const float ok[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          fold_state<4>(M, sum, acc, l[i], ok);
        }
      }
    }
    const float lse_nat = fold_finish<4>(M, sum, acc);
    const int tok = x >> group_shift;
    const int h = mi.kv_head * g + (x & (g - 1));
    const int64_t row = static_cast<int64_t>(mi.q_row0 + tok) * num_qo_heads + h;
    *reinterpret_cast<uint2*>(out + row * D + d0) =
        make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    if (lse_out != nullptr && d0 == 0) lse_out[row] = lse_nat;
  }
}

// bia_merge_states: (row, head) pairs, D/4 threads each.
template <int D>
__global__ void __launch_bounds__(kThreads)
merge_states_kernel(const float* __restrict__ v, const float* __restrict__ s,
                    const int32_t* __restrict__ indptr, int n_rows, int num_heads,
                    uint16_t* __restrict__ out, float* __restrict__ out_lse) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kThreads / TPR;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
  if (pair >= static_cast<int64_t>(n_rows) * num_heads) return;
  const int row = static_cast<int>(pair / num_heads);
  const int h = static_cast<int>(pair % num_heads);
  const int d0 = (threadIdx.x % TPR) * 4;
  float M = kNegInf, sum = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int lo = indptr[row], hi = indptr[row + 1];
  for (int k = lo; k < hi; ++k) {
    const int64_t st = static_cast<int64_t>(k) * num_heads + h;
    const float4 w = *reinterpret_cast<const float4*>(v + st * D + d0);
    const float ok[4] = {w.x, w.y, w.z, w.w};
    fold_state<4>(M, sum, acc, s[st], ok);
  }
  const float lse_nat = fold_finish<4>(M, sum, acc);
  *reinterpret_cast<uint2*>(out + pair * D + d0) =
      make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  if (out_lse != nullptr && d0 == 0) out_lse[pair] = lse_nat;
}

// ---------------------------------------------------------------------------
// KV append: one workgroup per AppendItem copies up to 16 new tokens (all kv
// heads, K and V) of one request from the packed k_new / v_new rows into
// their page slots. 16-byte copies; a token's Hkv * D row is contiguous on
// both sides.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
append_kernel(const bia::AppendItem* __restrict__ items, const uint16_t* __restrict__ k_new,
              const uint16_t* __restrict__ v_new, const int32_t* __restrict__ page_table,
              int row_elems, uint16_t* __restrict__ kp, uint16_t* __restrict__ vp) {
  const bia::AppendItem a = items[blockIdx.x];
  const int chunks = row_elems / 8;  // 16-byte pieces per token row
  for (int e = threadIdx.x; e < a.n_tok * chunks; e += kThreads) {
    const int t = e / chunks;
    const int c = e % chunks;
    const int pos = a.dst_pos0 + t;
    const int64_t page = page_table[a.page_off + (pos >> 4)];
    const int64_t dst = (page * 16 + (pos & 15)) * row_elems + c * 8;
    const int64_t src = static_cast<int64_t>(a.src_row0 + t) * row_elems + c * 8;
    *reinterpret_cast<uint4*>(kp + dst) = *reinterpret_cast<const uint4*>(k_new + src);
    *reinterpret_cast<uint4*>(vp + dst) = *reinterpret_cast<const uint4*>(v_new + src);
  }
}

// ---------------------------------------------------------------------------
// Device planner of the fixed-capacity (graph-capturable) decode. Workgroup r
// reads request r's kv_len from the device kv_indptr, sums the page counts of
// the requests before it for its page offset, checks the request, and writes
// its work items and merges in the form the host planner gives them. Kv head
// h's partition s keeps its partial states at slots
// ((r * Hkv + h) * max_splits + s) * g + head-in-group; the request's merge is
// at r * Hkv + h.
//
// Launch order: the host planner's, computed from kv_indptr alone by every
// workgroup. First the whole partitions of all requests in (request, kv
// head, partition) order, packed (request r's start after the whole
// partitions of the requests before it), then the requests' partial last
// partitions, longest first (ties by request index, then kv head), then the
// empty slots (n_tok = 0: the decode kernel returns at once).
//
// flags[r] is 0 for a valid request, else a reason bit. An invalid request
// reads no keys: the first of its slots gets an item with kv_len = 0 (its rows
// come out as the empty state, o = 0 and lse = -inf) and the rest are empty.
// Its slots are reserved from kv_len alone (one slot if kv_len itself is out
// of range), which every workgroup can compute.
// ---------------------------------------------------------------------------
constexpr int32_t kGraphBadKvLen = 1;  // kv_len < 1 or > max_kv_len
constexpr int32_t kGraphBadTable = 2;  // pages past page_table_capacity
constexpr int32_t kGraphBadPage = 4;   // a page id outside [0, num_pages)

__global__ void __launch_bounds__(kThreads)
decode_graph_plan_kernel(const int32_t* __restrict__ kv_indptr,
                         const int32_t* __restrict__ page_table, int num_kv_heads, int group,
                         int split, int max_splits, int max_kv_len, int num_pages,
                         int page_table_capacity, int32_t* __restrict__ flags,
                         WorkItem* __restrict__ items, MergeItem* __restrict__ merges) {
  __shared__ int64_t sm_red[5][kThreads];
  __shared__ int32_t sm_bad;
  const int r = blockIdx.x;
  const int batch = gridDim.x;
  const int tid = threadIdx.x;
  // slots request q reserves: nf whole partitions and np (0 or 1) partial one.
  // A valid kv_len fits 32 bits; 32-bit division is a few instructions where
  // the 64-bit one is a long software sequence
  auto reserve = [&](int q, int32_t& nf, int32_t& np) {
    const int64_t len = static_cast<int64_t>(kv_indptr[q + 1]) - kv_indptr[q];
    if (len < 1 || len > max_kv_len) {
      nf = 0;
      np = 1;
    } else {
      const int32_t l = static_cast<int32_t>(len);
      nf = l / split;
      np = l - nf * split != 0 ? 1 : 0;
    }
  };
  // 64-key tiles of request q's partial partition (0 when its slot holds the
  // empty state of an invalid request): partial partitions go longest first
  auto partial_tiles = [&](int q) -> int64_t {
    const int64_t len = static_cast<int64_t>(kv_indptr[q + 1]) - kv_indptr[q];
    if (len < 1 || len > max_kv_len) return 0;
    const int32_t l = static_cast<int32_t>(len);
    return (l - (l / split) * split + 63) / 64;
  };
  const int64_t my_tiles = partial_tiles(r);
  // integer sums over the requests (exact in any order): pages before r, whole
  // partitions of all and of the requests before r, partial partitions of all
  // and of those launched before r's (more tiles, or as many and an earlier
  // request)
  int64_t pages_before = 0, all_nf = 0, all_np = 0, np_before = 0, nf_before = 0;
  for (int q = tid; q < batch; q += kThreads) {
    const int64_t len = static_cast<int64_t>(kv_indptr[q + 1]) - kv_indptr[q];
    int32_t nf, np;
    reserve(q, nf, np);
    all_nf += nf;
    all_np += np;
    if (q < r) {
      pages_before += len > 0 ? (len + 15) / 16 : 0;
      nf_before += nf;
    }
    if (np != 0) {
      const int64_t tq = partial_tiles(q);
      if (tq > my_tiles || (tq == my_tiles && q < r)) np_before += 1;
    }
  }
  sm_red[0][tid] = pages_before;
  sm_red[1][tid] = all_nf;
  sm_red[2][tid] = all_np;
  sm_red[3][tid] = np_before;
  sm_red[4][tid] = nf_before;
  if (tid == 0) sm_bad = 0;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
#pragma unroll
      for (int k = 0; k < 5; ++k) sm_red[k][tid] += sm_red[k][tid + w];
    }
    __syncthreads();
  }
  const int64_t page_off = sm_red[0][0];
  const int64_t n_full = sm_red[1][0];        // whole-partition units of the launch
  const int64_t n_used = n_full + sm_red[2][0];
  const int64_t my_partial_unit = n_full + sm_red[3][0];
  const int64_t my_full_unit0 = sm_red[4][0];  // r's whole partitions start here

  const int64_t kv_len = static_cast<int64_t>(kv_indptr[r + 1]) - kv_indptr[r];
  int32_t bad = 0;
  if (kv_len < 1 || kv_len > max_kv_len) bad = kGraphBadKvLen;
  const int64_t n_pages = bad ? 0 : (kv_len + 15) / 16;
  if (!bad && page_off + n_pages > page_table_capacity) bad = kGraphBadTable;
  if (!bad) {
    bool any = false;
    // unrolled so that a long request's page-id loads are in flight together
#pragma unroll 8
    for (int64_t i = tid; i < n_pages; i += kThreads) {
      const int32_t pid = page_table[page_off + i];
      any = any || pid < 0 || pid >= num_pages;
    }
    if (any) sm_bad = kGraphBadPage;  // every writer stores the same value
  }
  __syncthreads();
  if (!bad) bad = sm_bad;
  if (tid == 0) flags[r] = bad;

  int32_t nf_r, np_r;
  reserve(r, nf_r, np_r);
  const int32_t n_res = nf_r + np_r;          // this request's partitions (= its slots)
  const int32_t n_splits = bad ? 0 : n_res;
  for (int sp = tid; sp < n_res; sp += kThreads) {
#pragma unroll 1
    for (int h = 0; h < num_kv_heads; ++h) {
      // whole partition sp of kv head h: (request, kv head, partition) order;
      // the partial one: its rank among the partial partitions
      const int64_t idx = sp < nf_r ? (my_full_unit0 * num_kv_heads +
                                       static_cast<int64_t>(h) * nf_r + sp)
                                    : my_partial_unit * num_kv_heads + h;
      WorkItem w{r, 0, 0, 0, 0, h, 0, -1};
      if (bad) {
        w.n_tok = sp == 0 ? 1 : 0;  // kv_len 0: the empty state
      } else {
        const int64_t slot = (static_cast<int64_t>(r) * num_kv_heads + h) * max_splits + sp;
        w.n_tok = 1;
        w.pos0 = static_cast<int32_t>(kv_len - 1);
        w.kv_len = static_cast<int32_t>(kv_len);
        w.page_off = static_cast<int32_t>(page_off);
        w.kv_begin = sp * split;
        w.state = n_splits > 1 ? static_cast<int32_t>(slot * group) : -1;
      }
      items[idx] = w;
    }
  }
  // this workgroup's share of the empty slots after the used ones
  const int64_t n_units = static_cast<int64_t>(batch) * max_splits;
  for (int64_t u = n_used + r + static_cast<int64_t>(tid) * batch; u < n_units;
       u += static_cast<int64_t>(kThreads) * batch) {
    for (int h = 0; h < num_kv_heads; ++h) items[u * num_kv_heads + h] = WorkItem{r, 0, 0, 0, 0, h, 0, -1};
  }
  for (int h = tid; h < num_kv_heads; h += kThreads) {
    const int64_t base = (static_cast<int64_t>(r) * num_kv_heads + h) * max_splits * group;
    merges[static_cast<int64_t>(r) * num_kv_heads + h] =
        MergeItem{static_cast<int32_t>(base), n_splits > 1 ? n_splits : 0, r,
                  n_splits > 1 ? 1 : 0, h, group, 0, 0};
  }
}

// ---------------------------------------------------------------------------
// Launch layer.
// ---------------------------------------------------------------------------
bia_status hip_fail(hipError_t e, const char* what) {
  return bia::fail(BIA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// ---------------------------------------------------------------------------
// Pinned work-list blocks. A plan takes one block from this library-owned
// pool when it is made and gives it back when it is destroyed, so run calls
// allocate nothing and destroying a plan never waits for the device. Each
// block is mapped and coherent (the upload kernel reads it over the bus
// without caching, so a reused block never returns stale lines) and carries
// an event recorded on the run's stream right after the upload that reads
// it: a returned block is handed out again only once that event has
// completed, i.e. once the device has passed every upload that read it.
// The event is created without the system-scope fence: it only reports
// progress (the upload's reads are over once the kernel has finished) and
// orders another stream of the same device behind it, and neither needs
// the device's caches written back for the host. With the fence, recording
// it left the device idle for about 3 us before the next kernel of every
// run call.
// Blocks are never freed before the process ends (hipHostFree would
// synchronise the device).
// ---------------------------------------------------------------------------
struct bia::PinBlock {
  void* host = nullptr;
  void* dev = nullptr;            // the same memory as the device addresses it
  size_t bytes = 0;               // capacity (a power of two)
  hipEvent_t done = nullptr;      // recorded after each upload from the block
  hipStream_t last_stream = nullptr;
  bool recorded = false;
};

namespace {

struct PinPool {
  std::mutex mu;
  std::vector<bia::PinBlock*> free_blocks;  // ready to hand out
  std::vector<bia::PinBlock*> returned;     // given back; may still be read
};
PinPool g_pin_pool;

constexpr size_t kPinMinBytes = 4096;

// Moves returned blocks whose last upload has completed to the free list
// (hipEventQuery does not wait). Caller holds the pool's mutex.
void pin_reclaim(PinPool& pool) {
  size_t keep = 0;
  for (size_t i = 0; i < pool.returned.size(); ++i) {
    bia::PinBlock* b = pool.returned[i];
    if (!b->recorded || hipEventQuery(b->done) == hipSuccess) {
      b->recorded = false;
      b->last_stream = nullptr;
      pool.free_blocks.push_back(b);
    } else {
      pool.returned[keep++] = b;
    }
  }
  pool.returned.resize(keep);
}

// A block of at least `bytes`, from the pool or newly pinned.
bia_status pin_acquire(size_t bytes, bia::PinBlock** out) {
  *out = nullptr;
  size_t cap = kPinMinBytes;
  while (cap < bytes) cap <<= 1;
  {
    std::lock_guard<std::mutex> lock(g_pin_pool.mu);
    pin_reclaim(g_pin_pool);
    bia::PinBlock* best = nullptr;
    size_t best_i = 0;
    for (size_t i = 0; i < g_pin_pool.free_blocks.size(); ++i) {
      bia::PinBlock* b = g_pin_pool.free_blocks[i];
      if (b->bytes >= cap && (best == nullptr || b->bytes < best->bytes)) {
        best = b;
        best_i = i;
      }
    }
    if (best != nullptr) {
      g_pin_pool.free_blocks.erase(g_pin_pool.free_blocks.begin() + best_i);
      *out = best;
      return BIA_OK;
    }
  }
  auto* b = new (std::nothrow) bia::PinBlock();
  if (b == nullptr) return bia::fail(BIA_ERR_INVALID_ARG, "out of host memory");
  hipError_t e = hipHostMalloc(&b->host, cap,
                               hipHostMallocMapped | hipHostMallocCoherent |
                                   hipHostMallocPortable);
  if (e != hipSuccess) {
    delete b;
    return hip_fail(e, "hipHostMalloc(work list)");
  }
  e = hipHostGetDevicePointer(&b->dev, b->host, 0);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&b->done, hipEventDisableTiming | hipEventDisableSystemFence);
  if (e != hipSuccess) {
    // a block that cannot be used stays out of the pool (never freed: no
    // synchronising call on this path either)
    delete b;
    return hip_fail(e, "work-list block set-up");
  }
  b->bytes = cap;
  *out = b;
  return BIA_OK;
}

void pin_release(bia::PinBlock* b) {
  if (b == nullptr) return;
  std::lock_guard<std::mutex> lock(g_pin_pool.mu);
  g_pin_pool.returned.push_back(b);
}

bool gpu_visible() {
  int n = 0;
  return hipGetDeviceCount(&n) == hipSuccess && n > 0;
}

// Work-list upload as a kernel on the run's stream (no copy-engine handoff
// before the kernels that read it): 16-byte words, grid-stride.
__global__ void __launch_bounds__(kThreads) upload_kernel(const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads)
    dst[i] = src[i];
}

// log2 of a power-of-two group (GQA 1..8, latent head blocks up to 128)
int log2_exact(int g) {
  int s = 0;
  while ((1 << s) < g) ++s;
  return s;
}

bia_status check_run(const bia_plan* plan, bia_mode mode, bool mla, const void* q, const void* k_pool,
                     const void* v_pool, const int32_t* page_table_dev, float sm_scale,
                     const void* out, const void* workspace, size_t workspace_bytes) {
  if (plan == nullptr) return bia::fail(BIA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->d.mode != mode)
    return bia::fail(BIA_ERR_INVALID_ARG, "plan was made for the other mode");
  if (plan->d.mla != mla)
    return bia::fail(BIA_ERR_INVALID_ARG, mla ? "plan was not made with BIA_PLAN_MLA"
                                              : "an MLA plan runs through bia_mla_*_paged");
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return bia::fail(BIA_ERR_INVALID_ARG, "sm_scale must be finite and positive");
  if (plan->d.items.empty()) return BIA_OK;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || page_table_dev == nullptr ||
      out == nullptr)
    return bia::fail(BIA_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (workspace == nullptr || workspace_bytes < plan->d.ws_bytes)
    return bia::fail(BIA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed",
                     workspace == nullptr ? size_t(0) : workspace_bytes, plan->d.ws_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % bia::kWsAlign != 0)
    return bia::fail(BIA_ERR_WORKSPACE, "workspace is not %zu-byte aligned", bia::kWsAlign);
  return BIA_OK;
}

// Copies the plan's work list from its pinned block into the head of the
// workspace on `stream`, then records the block's event. A block last read
// on another stream is waited for on this one first (no host wait), so the
// event always covers every upload that has read the block.
bia_status upload(const bia_plan* plan, void* workspace, hipStream_t stream) {
  const size_t bytes = plan->d.blob_bytes;
  if (bytes == 0) return BIA_OK;
  bia::PinBlock* b = plan->pin;
  if (b == nullptr)
    return bia::fail(BIA_ERR_HIP, "the plan holds no pinned work list (no GPU was visible "
                                  "when it was made)");
  hipError_t e = hipSuccess;
  if (b->recorded && b->last_stream != stream) {
    e = hipStreamWaitEvent(stream, b->done, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(work list)");
  }
  if (bytes % 16 != 0) {  // every list entry is 16 or 32 bytes
    e = hipMemcpyAsync(workspace, b->host, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work list)");
  } else {
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const unsigned grid =
        static_cast<unsigned>(std::min<int64_t>((n + kThreads - 1) / kThreads, 1024));
    hipLaunchKernelGGL(upload_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(b->dev), static_cast<uint4*>(workspace), n);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "work-list upload launch");
  }
  e = hipEventRecord(b->done, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(work list)");
  b->recorded = true;
  b->last_stream = stream;
  return BIA_OK;
}

// Where a decode or merge launch finds its work list and partial states.
struct ListLaunch {
  const unsigned char* items;  // WorkItem[] or MergeItem[] in the workspace
  unsigned n;                  // workgroups to launch
  int num_qo_heads, num_kv_heads, group, split;
  float* o_part;
  float* lse_part;
};

ListLaunch plan_items(const bia::PlanData& d, unsigned char* ws) {
  return ListLaunch{ws + d.off_items, static_cast<unsigned>(d.items.size()), d.num_qo_heads,
                    d.num_kv_heads, d.group, d.split, reinterpret_cast<float*>(ws + d.off_o),
                    reinterpret_cast<float*>(ws + d.off_lse)};
}

ListLaunch plan_merges(const bia::PlanData& d, unsigned char* ws) {
  ListLaunch L = plan_items(d, ws);
  L.items = ws + d.off_merges;
  L.n = static_cast<unsigned>(d.merges.size());
  return L;
}

// max_rows bounds the rows of one merge item: a prefill tile (tile tokens
// x group) or one decode token's group.
template <int D>
void launch_merge_tiles(const ListLaunch& L, int max_rows, uint16_t* out, float* lse,
                        hipStream_t stream) {
  constexpr int RPB = kThreads / (D / 4);
  const unsigned chunks = static_cast<unsigned>((max_rows + RPB - 1) / RPB);
  hipLaunchKernelGGL(merge_tiles_kernel<D>, dim3(L.n, chunks), dim3(kThreads), 0, stream,
                     reinterpret_cast<const MergeItem*>(L.items), L.o_part, L.lse_part,
                     L.num_qo_heads, log2_exact(L.group), out, lse);
}

int merge_rows(const bia::PlanData& d) {
  return (d.mode == BIA_MODE_DECODE ? 1 : d.tile_tokens) * d.group;
}

template <int D, int G>
void launch_decode(const ListLaunch& L, const uint16_t* q, const uint16_t* kp, const uint16_t* vp,
                   const int32_t* pt, float scale_log2, uint16_t* out, float* lse,
                   hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(L.n), dim3(kThreads), 0, stream,
                     reinterpret_cast<const WorkItem*>(L.items), q, kp, vp, pt, scale_log2,
                     L.num_qo_heads, L.num_kv_heads, L.split, out, lse, L.o_part, L.lse_part);
}

template <int D, int G>
void launch_decode_mfma(const ListLaunch& L, const uint16_t* q, const uint16_t* kp,
                        const uint16_t* vp, const int32_t* pt, float scale_log2, uint16_t* out,
                        float* lse, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mfma_kernel<D, G>), dim3(L.n), dim3(64 * kDecMfmaWaves), 0, stream,
                     reinterpret_cast<const WorkItem*>(L.items), q, kp, vp, pt, scale_log2,
                     L.num_qo_heads, L.num_kv_heads, L.split, out, lse, L.o_part, L.lse_part);
}

template <int D>
void launch_decode_g(const ListLaunch& L, const uint16_t* q, const uint16_t* kp,
                     const uint16_t* vp, const int32_t* pt, float scale_log2, uint16_t* out,
                     float* lse, hipStream_t stream) {
  // splits the LDS page list holds: the MFMA decode (the choice depends on
  // the split only, never on the batch)
  if (L.split <= 16 * kDecMfmaMaxPages) {
    switch (L.group) {
      case 1: launch_decode_mfma<D, 1>(L, q, kp, vp, pt, scale_log2, out, lse, stream); break;
      case 2: launch_decode_mfma<D, 2>(L, q, kp, vp, pt, scale_log2, out, lse, stream); break;
      case 4: launch_decode_mfma<D, 4>(L, q, kp, vp, pt, scale_log2, out, lse, stream); break;
      default: launch_decode_mfma<D, 8>(L, q, kp, vp, pt, scale_log2, out, lse, stream); break;
    }
    return;
  }
  switch (L.group) {
    case 1: launch_decode<D, 1>(L, q, kp, vp, pt, scale_log2, out, lse, stream); break;
    case 2: launch_decode<D, 2>(L, q, kp, vp, pt, scale_log2, out, lse, stream); break;
    case 4: launch_decode<D, 4>(L, q, kp, vp, pt, scale_log2, out, lse, stream); break;
    default: launch_decode<D, 8>(L, q, kp, vp, pt, scale_log2, out, lse, stream); break;
  }
}

}  // namespace

extern "C" bia_status bia_plan_create(bia_mode mode, const int32_t* qo_indptr,
                                      const int32_t* kv_indptr, const int32_t* page_table,
                                      int32_t batch, int32_t num_qo_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t page_size, int32_t num_pages,
                                      int32_t split_size, uint32_t flags,
                                      bia_plan** out_plan) {
  bia_status st = bia::plan_create_host(mode, qo_indptr, kv_indptr, page_table, batch,
                                        num_qo_heads, num_kv_heads, head_dim, page_size,
                                        num_pages, split_size, flags, out_plan);
  if (st != BIA_OK) return st;
  bia_plan* plan = *out_plan;
  // The pinned copy of the work list is made here, never in a run call. A
  // process that sees no GPU gets a plan it can inspect but not run.
  if (plan->d.blob_bytes == 0 || !gpu_visible()) return BIA_OK;
  st = pin_acquire(plan->d.blob_bytes, &plan->pin);
  if (st != BIA_OK) {
    bia::plan_free_host(plan);
    *out_plan = nullptr;
    return st;
  }
  std::memcpy(plan->pin->host, plan->d.blob.data(), plan->d.blob_bytes);
  return BIA_OK;
}

extern "C" void bia_plan_destroy(bia_plan* plan) {
  if (plan == nullptr) return;
  pin_release(plan->pin);  // reused only after its last upload has run
  bia::plan_free_host(plan);
}

extern "C" bia_status bia_prefill_paged(const bia_plan* plan, const void* q, const void* k_pool,
                                        const void* v_pool, const int32_t* page_table_dev,
                                        float sm_scale, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream_handle) {
  bia_status st = check_run(plan, BIA_MODE_PREFILL, false, q, k_pool, v_pool, page_table_dev, sm_scale,
                            out, workspace, workspace_bytes);
  if (st != BIA_OK || plan->d.items.empty()) return st;
  const bia::PlanData& d = plan->d;
  hipStream_t stream = static_cast<hipStream_t>(stream_handle);
  st = upload(plan, workspace, stream);
  if (st != BIA_OK) return st;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const float scale_log2 = sm_scale * kLog2e;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kp = static_cast<const uint16_t*>(k_pool);
  const auto* vp = static_cast<const uint16_t*>(v_pool);
  auto* o = static_cast<uint16_t*>(out);
  const auto* items = reinterpret_cast<const WorkItem*>(ws + d.off_items);
  auto* o_part = reinterpret_cast<float*>(ws + d.off_o);
  auto* lse_part = reinterpret_cast<float*>(ws + d.off_lse);
  const dim3 grid(static_cast<unsigned>(d.items.size()));
  if (d.head_dim == 128) {
    hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(kThreads), 0, stream, items, qq, kp, vp,
                       page_table_dev, scale_log2, d.num_qo_heads, d.num_kv_heads,
                       log2_exact(d.group), d.split, o, lse, o_part, lse_part);
  } else {
    hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(kThreads), 0, stream, items, qq, kp, vp,
                       page_table_dev, scale_log2, d.num_qo_heads, d.num_kv_heads,
                       log2_exact(d.group), d.split, o, lse, o_part, lse_part);
  }
  if (!d.merges.empty()) {
    if (d.head_dim == 128)
      launch_merge_tiles<128>(plan_merges(d, ws), merge_rows(d), o, lse, stream);
    else
      launch_merge_tiles<64>(plan_merges(d, ws), merge_rows(d), o, lse, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return BIA_OK;
}

namespace {

// Decode of a planned batch with the workspace at `workspace` (the caller's
// buffer, or the static one below).
bia_status run_decode(const bia_plan* plan, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* page_table_dev, float sm_scale,
                      void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream_handle) {
  const bia::PlanData& d = plan->d;
  hipStream_t stream = static_cast<hipStream_t>(stream_handle);
  bia_status st = upload(plan, workspace, stream);
  if (st != BIA_OK) return st;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const float scale_log2 = sm_scale * kLog2e;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kp = static_cast<const uint16_t*>(k_pool);
  const auto* vp = static_cast<const uint16_t*>(v_pool);
  auto* o = static_cast<uint16_t*>(out);
  if (d.head_dim == 128)
    launch_decode_g<128>(plan_items(d, ws), qq, kp, vp, page_table_dev, scale_log2, o, lse,
                         stream);
  else
    launch_decode_g<64>(plan_items(d, ws), qq, kp, vp, page_table_dev, scale_log2, o, lse,
                        stream);
  if (!d.merges.empty()) {
    if (d.head_dim == 128)
      launch_merge_tiles<128>(plan_merges(d, ws), merge_rows(d), o, lse, stream);
    else
      launch_merge_tiles<64>(plan_merges(d, ws), merge_rows(d), o, lse, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return BIA_OK;
}

// Workspace of bia_decode_paged_static: a file-scope device array, one copy
// per GPU, held until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: the kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up on the
// entry point's first call on that device and kept per device.
constexpr size_t kStaticWsBytes = BIA_STATIC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticWsBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

bia_status static_workspace(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return bia::fail(BIA_ERR_UNSUPPORTED, "device %d outside the %d the static workspace "
                                          "table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(static workspace)");
    if (ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % bia::kWsAlign != 0)
      return bia::fail(BIA_ERR_HIP, "static workspace address %p is not %zu-byte aligned",
                       ptr, bia::kWsAlign);
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return BIA_OK;
}

}  // namespace

extern "C" bia_status bia_decode_paged(const bia_plan* plan, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* page_table_dev,
                                       float sm_scale, void* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream_handle) {
  bia_status st = check_run(plan, BIA_MODE_DECODE, false, q, k_pool, v_pool, page_table_dev, sm_scale,
                            out, workspace, workspace_bytes);
  if (st != BIA_OK || plan->d.items.empty()) return st;
  return run_decode(plan, q, k_pool, v_pool, page_table_dev, sm_scale, out, lse, workspace,
                    workspace_bytes, stream_handle);
}

extern "C" bia_status bia_decode_paged_static(const bia_plan* plan, const void* q,
                                              const void* k_pool, const void* v_pool,
                                              const int32_t* page_table_dev, float sm_scale,
                                              void* out, float* lse, void* stream_handle) {
  if (plan != nullptr && plan->d.ws_bytes > kStaticWsBytes)
    return bia::fail(BIA_ERR_WORKSPACE,
                     "plan needs %zu bytes of workspace, above the %zu-byte static workspace",
                     plan->d.ws_bytes, kStaticWsBytes);
  // the checks of bia_decode_paged, with a stand-in for the workspace (its
  // address is looked up only once the call is known to run)
  bia_status st = check_run(plan, BIA_MODE_DECODE, false, q, k_pool, v_pool, page_table_dev,
                            sm_scale, out, reinterpret_cast<void*>(bia::kWsAlign),
                            kStaticWsBytes);
  if (st != BIA_OK || plan->d.items.empty()) return st;
  void* ws = nullptr;
  st = static_workspace(&ws);
  if (st != BIA_OK) return st;
  return run_decode(plan, q, k_pool, v_pool, page_table_dev, sm_scale, out, lse, ws,
                    kStaticWsBytes, stream_handle);
}

namespace {

bia_status run_mla(const bia_plan* plan, bia_mode mode, const void* q, const void* kv_pool,
                   const int32_t* page_table_dev, float sm_scale, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream_handle) {
  bia_status st = check_run(plan, mode, true, q, kv_pool, kv_pool, page_table_dev, sm_scale, out,
                            workspace, workspace_bytes);
  if (st != BIA_OK || plan->d.items.empty()) return st;
  const bia::PlanData& d = plan->d;
  hipStream_t stream = static_cast<hipStream_t>(stream_handle);
  st = upload(plan, workspace, stream);
  if (st != BIA_OK) return st;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const ListLaunch L = plan_items(d, ws);
  auto* o = static_cast<uint16_t*>(out);
  int hb_shift = 0;
  while ((1 << hb_shift) < d.group) ++hb_shift;
  if (mode == BIA_MODE_DECODE && d.group <= 16 && d.split <= 16 * kMlaDecMaxPages) {
    hipLaunchKernelGGL(mla_decode_kernel, dim3((L.n + kMlaDecWaves - 1) / kMlaDecWaves),
                       dim3(64 * kMlaDecWaves), 0, stream,
                       reinterpret_cast<const WorkItem*>(L.items), static_cast<int>(L.n),
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_pool),
                       page_table_dev, sm_scale * kLog2e, d.num_qo_heads, d.group, d.split, o,
                       lse, L.o_part, L.lse_part);
  } else {
    hipLaunchKernelGGL(mla_kernel, dim3(L.n), dim3(kMlaThreads), 0, stream,
                       reinterpret_cast<const WorkItem*>(L.items), static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(kv_pool), page_table_dev, sm_scale * kLog2e,
                       d.num_qo_heads, hb_shift, d.split, o, lse, L.o_part, L.lse_part);
  }
  if (!d.merges.empty()) {
    launch_merge_tiles<kMlaDv>(plan_merges(d, ws), merge_rows(d), o, lse, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "MLA launch");
  return BIA_OK;
}

}  // namespace

extern "C" bia_status bia_mla_prefill_paged(const bia_plan* plan, const void* q,
                                            const void* kv_pool, const int32_t* page_table_dev,
                                            float sm_scale, void* out, float* lse,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream_handle) {
  return run_mla(plan, BIA_MODE_PREFILL, q, kv_pool, page_table_dev, sm_scale, out, lse,
                 workspace, workspace_bytes, stream_handle);
}

extern "C" bia_status bia_mla_decode_paged(const bia_plan* plan, const void* q,
                                           const void* kv_pool, const int32_t* page_table_dev,
                                           float sm_scale, void* out, float* lse,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream_handle) {
  return run_mla(plan, BIA_MODE_DECODE, q, kv_pool, page_table_dev, sm_scale, out, lse,
                 workspace, workspace_bytes, stream_handle);
}

extern "C" bia_status bia_merge_states(const float* v, const float* s,
                                       const int32_t* state_indptr_dev, int32_t n_rows,
                                       int32_t num_heads, int32_t head_dim, void* out,
                                       float* out_lse, void* stream_handle) {
  if (n_rows < 0 || num_heads <= 0)
    return bia::fail(BIA_ERR_INVALID_ARG, "n_rows %d / num_heads %d out of range", n_rows,
                     num_heads);
  if (head_dim != 64 && head_dim != 128)
    return bia::fail(BIA_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)", head_dim);
  if (n_rows == 0) return BIA_OK;
  if (v == nullptr || s == nullptr || state_indptr_dev == nullptr || out == nullptr)
    return bia::fail(BIA_ERR_INVALID_ARG, "a required device pointer is NULL");
  hipStream_t stream = static_cast<hipStream_t>(stream_handle);
  const int64_t pairs = static_cast<int64_t>(n_rows) * num_heads;
  const int rpb = kThreads / (head_dim / 4);
  const int64_t blocks = (pairs + rpb - 1) / rpb;
  if (blocks > INT32_MAX) return bia::fail(BIA_ERR_SHAPE, "too many rows to merge");
  auto* o = static_cast<uint16_t*>(out);
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_states_kernel<128>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, v, s, state_indptr_dev, n_rows, num_heads, o,
                       out_lse);
  else
    hipLaunchKernelGGL(merge_states_kernel<64>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, v, s, state_indptr_dev, n_rows, num_heads, o,
                       out_lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return BIA_OK;
}

extern "C" bia_status bia_append_paged_kv(const bia_plan* plan, const void* k_new,
                                          const void* v_new, const int32_t* page_table_dev,
                                          void* k_pool, void* v_pool, void* workspace,
                                          size_t workspace_bytes, void* stream_handle) {
  if (plan == nullptr) return bia::fail(BIA_ERR_INVALID_ARG, "plan is NULL");
  const bia::PlanData& d = plan->d;
  if (d.mla)
    return bia::fail(BIA_ERR_UNSUPPORTED, "append into a latent (MLA) cache is not supported");
  if (d.appends.empty()) return BIA_OK;
  if (k_new == nullptr || v_new == nullptr || page_table_dev == nullptr || k_pool == nullptr ||
      v_pool == nullptr)
    return bia::fail(BIA_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (workspace == nullptr || workspace_bytes < d.ws_bytes)
    return bia::fail(BIA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed",
                     workspace == nullptr ? size_t(0) : workspace_bytes, d.ws_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % bia::kWsAlign != 0)
    return bia::fail(BIA_ERR_WORKSPACE, "workspace is not %zu-byte aligned", bia::kWsAlign);
  hipStream_t stream = static_cast<hipStream_t>(stream_handle);
  bia_status st = upload(plan, workspace, stream);
  if (st != BIA_OK) return st;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<unsigned>(d.appends.size())), dim3(kThreads),
                     0, stream, reinterpret_cast<const bia::AppendItem*>(ws + d.off_appends),
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                     page_table_dev, d.num_kv_heads * d.head_dim, static_cast<uint16_t*>(k_pool),
                     static_cast<uint16_t*>(v_pool));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return BIA_OK;
}

extern "C" bia_status bia_decode_graph_run(const bia_decode_graph* dg, int32_t batch,
                                           const int32_t* kv_indptr_dev, const void* q,
                                           const void* k_pool, const void* v_pool,
                                           const int32_t* page_table_dev, float sm_scale,
                                           void* out, float* lse, void* workspace,
                                           size_t workspace_bytes, void* stream_handle) {
  if (dg == nullptr) return bia::fail(BIA_ERR_INVALID_ARG, "decode graph handle is NULL");
  const bia::DecodeGraphData& d = dg->d;
  if (batch < 0 || batch > d.max_batch)
    return bia::fail(BIA_ERR_SHAPE, "batch %d outside [0, %d]", batch, d.max_batch);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return bia::fail(BIA_ERR_INVALID_ARG, "sm_scale must be finite and positive");
  if (batch == 0) return BIA_OK;
  if (kv_indptr_dev == nullptr || q == nullptr || k_pool == nullptr || v_pool == nullptr ||
      page_table_dev == nullptr || out == nullptr)
    return bia::fail(BIA_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (workspace == nullptr || workspace_bytes < d.ws_bytes)
    return bia::fail(BIA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed",
                     workspace == nullptr ? size_t(0) : workspace_bytes, d.ws_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % bia::kWsAlign != 0)
    return bia::fail(BIA_ERR_WORKSPACE, "workspace is not %zu-byte aligned", bia::kWsAlign);
  hipStream_t stream = static_cast<hipStream_t>(stream_handle);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  auto* flags = reinterpret_cast<int32_t*>(ws + d.off_flags);
  auto* items = reinterpret_cast<WorkItem*>(ws + d.off_items);
  auto* merges = reinterpret_cast<MergeItem*>(ws + d.off_merges);
  hipLaunchKernelGGL(decode_graph_plan_kernel, dim3(static_cast<unsigned>(batch)),
                     dim3(kThreads), 0, stream, kv_indptr_dev, page_table_dev, d.num_kv_heads,
                     d.group, d.split, d.max_splits, d.max_kv_len, d.num_pages,
                     d.page_table_capacity, flags, items, merges);
  ListLaunch L{ws + d.off_items,
               static_cast<unsigned>(int64_t(batch) * d.num_kv_heads * d.max_splits),
               d.num_qo_heads, d.num_kv_heads, d.group, d.split,
               reinterpret_cast<float*>(ws + d.off_o), reinterpret_cast<float*>(ws + d.off_lse)};
  const float scale_log2 = sm_scale * kLog2e;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kp = static_cast<const uint16_t*>(k_pool);
  const auto* vp = static_cast<const uint16_t*>(v_pool);
  auto* o = static_cast<uint16_t*>(out);
  if (d.head_dim == 128)
    launch_decode_g<128>(L, qq, kp, vp, page_table_dev, scale_log2, o, lse, stream);
  else
    launch_decode_g<64>(L, qq, kp, vp, page_table_dev, scale_log2, o, lse, stream);
  if (d.max_splits > 1) {
    L.items = ws + d.off_merges;
    L.n = static_cast<unsigned>(int64_t(batch) * d.num_kv_heads);
    if (d.head_dim == 128)
      launch_merge_tiles<128>(L, d.group, o, lse, stream);
    else
      launch_merge_tiles<64>(L, d.group, o, lse, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode graph launch");
  return BIA_OK;
}

extern "C" bia_status bia_decode_graph_read_flags(const bia_decode_graph* dg,
                                                  const void* workspace, int32_t batch,
                                                  int32_t* flags_host, void* stream_handle) {
  if (dg == nullptr || workspace == nullptr || flags_host == nullptr)
    return bia::fail(BIA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (batch < 0 || batch > dg->d.max_batch)
    return bia::fail(BIA_ERR_SHAPE, "batch %d outside [0, %d]", batch, dg->d.max_batch);
  if (batch == 0) return BIA_OK;
  hipStream_t stream = static_cast<hipStream_t>(stream_handle);
  const auto* src = static_cast<const unsigned char*>(workspace) + dg->d.off_flags;
  hipError_t e = hipMemcpyAsync(flags_host, src, size_t(batch) * sizeof(int32_t),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "reading decode graph flags");
  return BIA_OK;
}
