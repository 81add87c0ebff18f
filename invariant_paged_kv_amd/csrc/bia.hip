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
// Software pipeline (per wave): the score MFMAs of tile j+1 are issued in the
// same block as the softmax of tile j, so matrix and vector work overlap;
// K runs one tile ahead of V through single LDS buffers, refilled from
// registers loaded two tiles ahead from HBM (two barriers per tile).
//
// LDS: K and V both row-major, [64][D + 8] and [64][D + 16]. K rows are read
// 16 bytes per lane (the pad keeps 8 consecutive rows on distinct banks); the
// V^T operand comes from ds_read_b64_tr_b16: in each 16-lane group, lane i
// addresses 4 dims of key i / 4, and lane j = 4a + b receives dim 4a + b of
// those 4 keys (the 32-byte pad keeps the 4 rows on distinct banks).
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
// more than kLazyMax (base-2 units), so most tiles rescale nothing; scores
// are scaled inside the exponent (exp2(s * c - m)); masking runs only on
// tiles that reach past the wave's first row position (elsewhere every key
// is visible to every row of the wave). The row sum adds the fp32
// probabilities (summing their bf16 roundings would cost ~1e-3 in lse).
// ---------------------------------------------------------------------------
constexpr float kLazyMax = 8.0f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  // p points into __shared__ memory; the C-style cast moves it to the LDS
  // address space, which the transposing read requires.
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

// max over lanes l and l ^ 32
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(x, fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(r[0])),
                        __builtin_bit_cast(float, static_cast<unsigned>(r[1]))));
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
  constexpr int KS = D + 8;   // bf16 per K row in LDS
  constexpr int VS = D + 16;  // bf16 per V row in LDS
  constexpr int C = D / 8;    // 16-byte chunks per K/V row
  constexpr int NK = C / 4;   // consecutive keys one thread stages (4 or 2)
  constexpr int DB = D / 32;  // 32-wide d blocks of the output
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[64 * KS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[64 * VS];

  const WorkItem it = items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;
  const int col = lane & 31;
  const int g = 1 << group_shift;
  const int x = wave * 32 + col;  // this lane's row of the q tile
  const int tok = x >> group_shift;
  const int hj = x & (g - 1);
  const bool row_valid = tok < it.n_tok;
  const int pos = row_valid ? it.pos0 + tok : -1;
  // Position of the wave's first row: tiles ending at or before it need no mask.
  const int wave_pos0 = it.pos0 + ((wave * 32) >> group_shift);
  const int64_t q_off =
      (static_cast<int64_t>(it.q_row0 + tok) * num_qo_heads + it.kv_head * g + hj) * D;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row_valid) w = *reinterpret_cast<const uint4*>(q + q_off + 16 * s + 8 * hi);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }

  const int last = it.pos0 + it.n_tok - 1;
  const int kv_end = min(it.kv_begin + split, last + 1);
  const int n_tiles = (kv_end - it.kv_begin + 63) >> 6;
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * D;

  // Staging: this thread moves NK consecutive keys (one page: NK divides 16)
  // times 8 dims of K and V per tile.
  const int sc = tid % C;
  const int skey = (tid / C) * NK;
  const int64_t thread_off = static_cast<int64_t>(it.kv_head) * D + sc * 8;
  const int32_t* pt = page_table + it.page_off;
  uint4 kreg[NK], vreg[NK];

  auto page_of = [&](int t) -> int32_t {
    const int kk = it.kv_begin + 64 * t + skey;
    return kk < kv_end ? pt[kk >> 4] : 0;
  };
  auto fetch = [&](uint4 (&reg)[NK], const uint16_t* __restrict__ pool, int t,
                   int64_t page) {
    const int kk0 = it.kv_begin + 64 * t + skey;
    const uint16_t* b = pool + (page * 16 + (kk0 & 15)) * slot_stride + thread_off;
    if (kk0 + NK <= kv_end) {
#pragma unroll
      for (int e = 0; e < NK; ++e) reg[e] = *reinterpret_cast<const uint4*>(b + e * slot_stride);
    } else {  // ragged end of the item: keys at or past kv_end are zero
#pragma unroll
      for (int e = 0; e < NK; ++e) {
        reg[e] = make_uint4(0, 0, 0, 0);
        if (kk0 + e < kv_end) reg[e] = *reinterpret_cast<const uint4*>(b + e * slot_stride);
      }
    }
  };
  auto stash_k = [&]() {
#pragma unroll
    for (int e = 0; e < NK; ++e)
      *reinterpret_cast<uint4*>(&k_lds[(skey + e) * KS + sc * 8]) = kreg[e];
  };
  auto stash_v = [&]() {
#pragma unroll
    for (int e = 0; e < NK; ++e)
      *reinterpret_cast<uint4*>(&v_lds[(skey + e) * VS + sc * 8]) = vreg[e];
  };
  auto scores = [&](f32x16 (&acc)[2]) {
    acc[0] = f32x16{};
    acc[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 kw = *reinterpret_cast<const uint4*>(
            &k_lds[(32 * kb + col) * KS + 16 * s + 8 * hi]);
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kw), qf[s],
                                                          acc[kb], 0, 0, 0);
      }
    }
  };
  // This lane's base in v_lds for the transposed reads (see the header).
  const int v_lane = (((lane & 15) >> 2) + 4 * hi) * VS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  float m = kNegInf;  // running max (base-2 scaled logits), possibly stale by < kLazyMax
  float lsum = 0.0f;  // this lane-half's running sum of probabilities
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b] = f32x16{};

  // ---- prologue: K(0), V(0) in LDS; S = scores of tile 0; K(1) in LDS;
  // registers hold K(2) and V(1); page ids for V(2) and K(3) ready ----
  f32x16 sacc[2];
  {
    const int32_t p0 = page_of(0);
    const int32_t p1 = page_of(1);
    const int32_t p2 = page_of(2);
    fetch(kreg, kp, 0, p0);
    fetch(vreg, vp, 0, p0);
    stash_k();
    stash_v();
    if (n_tiles > 1) {
      fetch(kreg, kp, 1, p1);
      fetch(vreg, vp, 1, p1);
    }
    __syncthreads();
    scores(sacc);
    __syncthreads();
    if (n_tiles > 1) stash_k();
    if (n_tiles > 2) fetch(kreg, kp, 2, p2);
    __syncthreads();
  }
  int32_t page_v = page_of(2);  // page ids for V(j + 2) and K(j + 3)
  int32_t page_k = page_of(3);

  // One tile of the pipeline: softmax of `cur` (tile j) overlapped with the
  // score MFMAs of tile j+1 into `nxt` (when HasNext), then PV of tile j and
  // the LDS/register refills for the tiles after it.
  auto body = [&](auto has_next, f32x16 (&cur)[2], f32x16 (&nxt)[2], int j) {
    constexpr bool kHasNext = decltype(has_next)::value;
    const int t0 = it.kv_begin + 64 * j;
    if (t0 + 63 > wave_pos0) {  // wave-uniform: some key is past some row
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = t0 + 32 * kb + 8 * (v >> 2) + 4 * hi + (v & 3);
          cur[kb][v] = key <= pos ? cur[kb][v] : kNegInf;
        }
      }
    }
    if constexpr (kHasNext) scores(nxt);
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, cur[kb][v]);
    }
    mt = max_halves(mt) * scale_log2;
    const bool raise = mt > m + kLazyMax;  // true on the first tile with a visible key
    const float m_new = raise ? mt : m;
    const float alpha = raise ? fast_exp2(m - m_new) : 1.0f;
    const float neg_m = (m_new == kNegInf) ? 0.0f : -m_new;
    float psum = 0.0f;
    uint32_t pw[2][2][4];  // [kb][half][pair] packed bf16 probabilities
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(cur[kb][v], scale_log2, neg_m));
        const float p1 = fast_exp2(__builtin_fmaf(cur[kb][v + 1], scale_log2, neg_m));
        psum += p0;
        psum += p1;
        pw[kb][v >> 3][(v & 7) >> 1] = pack_bf16x2(p0, p1);
      }
    }
    if (__any(raise)) {  // lanes that did not raise have alpha == 1 exactly
      lsum *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= alpha;
    }
    lsum += psum;
    m = m_new;

    // Every wave is done reading K(j+1), and V(j), stored by all waves after
    // the previous tile's second barrier, is visible. The last tile needs the
    // barrier for the second reason alone.
    __syncthreads();
    if constexpr (kHasNext) {
      if (j + 2 < n_tiles) stash_k();
      if (j + 3 < n_tiles) fetch(kreg, kp, j + 3, page_k);
    }

    // ---- O^T += V^T P^T (V of tile j) ----
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint16_t* src = &v_lds[v_lane + (32 * kb + 16 * h) * VS + 32 * b];
          const uint2 lo = lds_read_tr16(src);
          const uint2 up = lds_read_tr16(src + 8 * VS);
          const uint4 va = make_uint4(lo.x, lo.y, up.x, up.y);
          const uint4 pb = make_uint4(pw[kb][h][0], pw[kb][h][1], pw[kb][h][2], pw[kb][h][3]);
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb), o[b], 0, 0, 0);
        }
      }
    }
    if constexpr (kHasNext) {
      __syncthreads();  // every wave is done reading V(j)
      stash_v();        // V(j+1)
      if (j + 2 < n_tiles) fetch(vreg, vp, j + 2, page_v);
      page_v = page_k;
      page_k = page_of(j + 4);
    }
  };

  // Unrolled by two so the score registers alternate without copies; the
  // last tile has no successor to prefetch.
  f32x16 sb[2];
  int j = 0;
  for (; j + 2 < n_tiles; j += 2) {
    body(std::true_type{}, sacc, sb, j);
    body(std::true_type{}, sb, sacc, j + 1);
  }
  if (j + 1 < n_tiles) {
    body(std::true_type{}, sacc, sb, j);
    body(std::false_type{}, sb, sacc, j + 1);
  } else {
    body(std::false_type{}, sacc, sb, j);
  }

  // ---- this partition's state for the row: o = O / l, lse = m + log l ----
  const float l_row = lsum + __shfl_xor(lsum, 32);
  if (!row_valid) return;
  float lse_nat = kNegInf;
  float inv = 0.0f;
  if (l_row > 0.0f) {
    inv = 1.0f / l_row;
    lse_nat = (m + fast_log2(l_row)) * kLn2;
  }
  if (it.state < 0) {
    uint16_t* orow = out + q_off;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d = 32 * b + 8 * v4 + 4 * hi;
        const uint2 w = make_uint2(pack_bf16x2(o[b][4 * v4] * inv, o[b][4 * v4 + 1] * inv),
                                   pack_bf16x2(o[b][4 * v4 + 2] * inv, o[b][4 * v4 + 3] * inv));
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
    }
    if (lse_out != nullptr && hi == 0)
      lse_out[static_cast<int64_t>(it.q_row0 + tok) * num_qo_heads + it.kv_head * g + hj] = lse_nat;
  } else {
    const int64_t st = static_cast<int64_t>(it.state) + x;
    float* orow = o_part + st * D;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d = 32 * b + 8 * v4 + 4 * hi;
        *reinterpret_cast<float4*>(orow + d) =
            make_float4(o[b][4 * v4] * inv, o[b][4 * v4 + 1] * inv, o[b][4 * v4 + 2] * inv,
                        o[b][4 * v4 + 3] * inv);
      }
    }
    if (hi == 0) lse_part[st] = lse_nat;
  }
}

// ---------------------------------------------------------------------------
// Decode: one workgroup = one WorkItem = (request, kv head, partition of up to
// `split` keys), g q heads. The partition's keys go in 16-key chunks to the 4
// waves round-robin (chunk c -> wave c % 4). In a wave, 8 lanes share one key
// (each holds D/8 of its dims, so 16-byte loads read whole rows) and a lane
// group takes keys c*16 + ks and c*16 + 8 + ks (one page). Chunks are double
// buffered in registers: the loads of a wave's next chunk are in flight
// while the current one is computed, and page ids are read a chunk earlier
// still.
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

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 2)
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
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  // page id of this lane group's keys in chunk c (both keys share a page)
  auto page_of = [&](int c) -> int32_t {
    const int key = it.kv_begin + CHUNK * c + ks;
    return (c < n_chunks && key < kv_end) ? pt[key >> 4] : 0;
  };
  auto load = [&](uint32_t (&kw)[2][W], uint32_t (&vw)[2][W], int c, int64_t page) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = it.kv_begin + CHUNK * c + 8 * i + ks;
      if (key < kv_end) {
        const int64_t off = (page * 16 + (key & 15)) * slot_stride + head_off;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint4 a = *reinterpret_cast<const uint4*>(kp + off + 8 * u);
          const uint4 b = *reinterpret_cast<const uint4*>(vp + off + 8 * u);
          kw[i][4 * u] = a.x; kw[i][4 * u + 1] = a.y; kw[i][4 * u + 2] = a.z; kw[i][4 * u + 3] = a.w;
          vw[i][4 * u] = b.x; vw[i][4 * u + 1] = b.y; vw[i][4 * u + 2] = b.z; vw[i][4 * u + 3] = b.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < W; ++u) {
          kw[i][u] = 0;
          vw[i][u] = 0;
        }
      }
    }
  };
  auto compute = [&](const uint32_t (&kw)[2][W], const uint32_t (&vw)[2][W], int c) {
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

  // This wave's chunks are wave, wave + 4, ...: two register buffers
  // alternate; page ids run one chunk ahead of the loads that use them.
  uint32_t ka[2][W], va[2][W], kb2[2][W], vb2[2][W];
  int c = wave;
  if (c < n_chunks) load(ka, va, c, page_of(c));
  int32_t page_next = page_of(c + 4);
  for (; c < n_chunks; c += 8) {
    if (c + 4 < n_chunks) load(kb2, vb2, c + 4, page_next);
    page_next = page_of(c + 8);
    compute(ka, va, c);
    if (c + 4 >= n_chunks) break;
    if (c + 8 < n_chunks) load(ka, va, c + 8, page_next);
    page_next = page_of(c + 12);
    compute(kb2, vb2, c + 4);
  }

  // ---- combine the 8 key groups of the wave (butterfly over lane ^ 8, 16, 32) ----
#pragma unroll
  for (int mask = 8; mask <= 32; mask <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float o2[DPL];
#pragma unroll
      for (int i = 0; i < DPL; ++i) o2[i] = __shfl_xor(o[j][i], mask);
      const float m2 = __shfl_xor(m[j], mask);
      const float l2 = __shfl_xor(l[j], mask);
      combine_sym<DPL>(m[j], l[j], o[j], m2, l2, o2);
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
  constexpr int RPP = kThreads / TPR;     // rows per pass
  const MergeItem mi = merges[blockIdx.x];
  const int g = 1 << group_shift;
  const int rows = mi.n_tok * g;
  const int d0 = (threadIdx.x % TPR) * 4;
  for (int x = threadIdx.x / TPR; x < rows; x += RPP) {
    float M = kNegInf, sum = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < mi.n_splits; ++k) {
      const int64_t st = static_cast<int64_t>(mi.state0) + static_cast<int64_t>(k) * mi.stride + x;
      const float4 v = *reinterpret_cast<const float4*>(o_part + st * D + d0);
      const float ok[4] = {v.x, v.y, v.z, v.w};
      fold_state<4>(M, sum, acc, lse_part[st], ok);
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
// Launch layer.
// ---------------------------------------------------------------------------
std::mutex g_pin_mutex;

bia_status hip_fail(hipError_t e, const char* what) {
  return bia::fail(BIA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Pinned host copy of the plan's work list, made once per plan so the
// per-run upload is a true async copy.
bia_status ensure_pinned(const bia_plan* plan) {
  std::lock_guard<std::mutex> lock(g_pin_mutex);
  bia_plan* p = const_cast<bia_plan*>(plan);
  if (p->pinned != nullptr || p->d.blob_bytes == 0) return BIA_OK;
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, p->d.blob_bytes, hipHostMallocDefault);
  if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(work list)");
  std::memcpy(h, p->d.blob.data(), p->d.blob_bytes);
  p->pinned = h;
  return BIA_OK;
}

int log2_exact(int g) { return g == 1 ? 0 : g == 2 ? 1 : g == 4 ? 2 : 3; }

bia_status check_run(const bia_plan* plan, bia_mode mode, const void* q, const void* k_pool,
                     const void* v_pool, const int32_t* page_table_dev, float sm_scale,
                     const void* out, const void* workspace, size_t workspace_bytes) {
  if (plan == nullptr) return bia::fail(BIA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->d.mode != mode)
    return bia::fail(BIA_ERR_INVALID_ARG, "plan was made for the other mode");
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

bia_status upload(const bia_plan* plan, void* workspace, hipStream_t stream) {
  bia_status st = ensure_pinned(plan);
  if (st != BIA_OK) return st;
  hipError_t e = hipMemcpyAsync(workspace, plan->pinned, plan->d.blob_bytes,
                                hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work list)");
  return BIA_OK;
}

template <int D>
void launch_merge_tiles(const bia::PlanData& d, unsigned char* ws, uint16_t* out, float* lse,
                        hipStream_t stream) {
  hipLaunchKernelGGL(merge_tiles_kernel<D>, dim3(static_cast<unsigned>(d.merges.size())),
                     dim3(kThreads), 0, stream,
                     reinterpret_cast<const MergeItem*>(ws + d.off_merges),
                     reinterpret_cast<const float*>(ws + d.off_o),
                     reinterpret_cast<const float*>(ws + d.off_lse), d.num_qo_heads,
                     log2_exact(d.group), out, lse);
}

template <int D, int G>
void launch_decode(const bia::PlanData& d, unsigned char* ws, const uint16_t* q,
                   const uint16_t* kp, const uint16_t* vp, const int32_t* pt, float scale_log2,
                   uint16_t* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(static_cast<unsigned>(d.items.size())),
                     dim3(kThreads), 0, stream,
                     reinterpret_cast<const WorkItem*>(ws + d.off_items), q, kp, vp, pt,
                     scale_log2, d.num_qo_heads, d.num_kv_heads, d.split, out, lse,
                     reinterpret_cast<float*>(ws + d.off_o),
                     reinterpret_cast<float*>(ws + d.off_lse));
}

template <int D>
void launch_decode_g(const bia::PlanData& d, unsigned char* ws, const uint16_t* q,
                     const uint16_t* kp, const uint16_t* vp, const int32_t* pt,
                     float scale_log2, uint16_t* out, float* lse, hipStream_t stream) {
  switch (d.group) {
    case 1: launch_decode<D, 1>(d, ws, q, kp, vp, pt, scale_log2, out, lse, stream); break;
    case 2: launch_decode<D, 2>(d, ws, q, kp, vp, pt, scale_log2, out, lse, stream); break;
    case 4: launch_decode<D, 4>(d, ws, q, kp, vp, pt, scale_log2, out, lse, stream); break;
    default: launch_decode<D, 8>(d, ws, q, kp, vp, pt, scale_log2, out, lse, stream); break;
  }
}

}  // namespace

extern "C" void bia_plan_destroy(bia_plan* plan) {
  if (plan == nullptr) return;
  if (plan->pinned != nullptr) (void)hipHostFree(plan->pinned);
  delete plan;
}

extern "C" bia_status bia_prefill_paged(const bia_plan* plan, const void* q, const void* k_pool,
                                        const void* v_pool, const int32_t* page_table_dev,
                                        float sm_scale, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream_handle) {
  bia_status st = check_run(plan, BIA_MODE_PREFILL, q, k_pool, v_pool, page_table_dev, sm_scale,
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
      launch_merge_tiles<128>(d, ws, o, lse, stream);
    else
      launch_merge_tiles<64>(d, ws, o, lse, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return BIA_OK;
}

extern "C" bia_status bia_decode_paged(const bia_plan* plan, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* page_table_dev,
                                       float sm_scale, void* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream_handle) {
  bia_status st = check_run(plan, BIA_MODE_DECODE, q, k_pool, v_pool, page_table_dev, sm_scale,
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
  if (d.head_dim == 128)
    launch_decode_g<128>(d, ws, qq, kp, vp, page_table_dev, scale_log2, o, lse, stream);
  else
    launch_decode_g<64>(d, ws, qq, kp, vp, page_table_dev, scale_log2, o, lse, stream);
  if (!d.merges.empty()) {
    if (d.head_dim == 128)
      launch_merge_tiles<128>(d, ws, o, lse, stream);
    else
      launch_merge_tiles<64>(d, ws, o, lse, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return BIA_OK;
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
