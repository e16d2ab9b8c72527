// Device-side definitions shared by the attention kernels (gfx950 / CDNA4).
//
// The mask predicates and score modifiers follow the FlexAttention write-up
// "新PyTorch API：几行代码实现不同注意力变体，兼具FlashAttention性能和PyTorch
// 灵活性": §FlexAttention (score_mod applied to every score before softmax,
// indexed by (b, h, q_idx, kv_idx)), §相对位置编码 (bias from the query-key
// distance computed in-kernel), §Causal Mask, §Sliding Window + Causal, and
// the PrefixLM / document-mask / ALiBi entries of its variant list.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn_fa2.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Kernel-side mask kind for SLIDING and DOCUMENT together (what any AND set
// holding both reduces to).  Internal only: never a value of the public enum.
constexpr int kMaskDocWindow = 6;

// Kernel-side copy of the mask parameters (plain values, passed by value);
// kind is NONE..DOCUMENT or kMaskDocWindow.
struct MaskArgs {
  int kind;
  int window;
  int prefix_len;
  const int32_t *doc_ids;  // [B, S]
  int doc_stride;          // S
};

// Kernel-side score-modifier parameters. For ALIBI the per-head slope is read
// from `slopes` or, when null, computed as 2^(-8 (h+1) / Hq).
struct ScoreArgs {
  int kind;
  const float *slopes;
  float rel_scale;
  float softcap;   // SOFTCAP: the cap, > 0
};

// visible(b, i, j) of the mask kind.  doc_i is doc_ids[b, i] (read once per
// query row by the caller); the key's id is read here only for DOCUMENT.
__device__ __forceinline__ bool mask_visible(const MaskArgs &m, int i, int j, int doc_i,
                                             const int32_t *doc_row) {
  switch (m.kind) {
    case ATTN_MASK_NONE: return true;
    case ATTN_MASK_CAUSAL: return j <= i;
    case ATTN_MASK_SLIDING: return (j <= i) && (i - j < m.window);
    case ATTN_MASK_PREFIX_LM: return (j <= i) || (j < m.prefix_len);
    case ATTN_MASK_DOCUMENT: return (j <= i) && (doc_row[j] == doc_i);
    case kMaskDocWindow: return (j <= i) && (i - j < m.window) && (doc_row[j] == doc_i);
    default: return false;
  }
}

// ALiBi slope of query head hq.
__device__ __forceinline__ float alibi_slope(const ScoreArgs &s, int hq, int Hq) {
  if (s.slopes) return s.slopes[hq];
  return exp2f(-8.0f * (float)(hq + 1) / (float)Hq);
}

// Coefficient a of the modifier written as a * (j - i): ALIBI a = slope,
// REL_POS a = -rel_scale (c * (i - j) = -c * (j - i)), NONE a = 0.
__device__ __forceinline__ float bias_coeff(const ScoreArgs &s, int hq, int Hq) {
  if (s.kind == ATTN_SCORE_ALIBI) return alibi_slope(s, hq, Hq);
  if (s.kind == ATTN_SCORE_REL_POS) return -s.rel_scale;
  return 0.0f;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Soft-capping of a log2-domain score x = s * log2(e): C tanh(x / C) with
// C = cap * log2(e), written as C - 2C / (1 + 2^(kx)), k = 2 / cap (since
// e^(2x/C) = 2^(2x/cap)).  k_scaled = k * c folds in a prior multiply x = c s.
// Saturates to +-C without overflow (2^(kx) = inf gives C, 0 gives -C).  The
// hardware exp2 and reciprocal leave an absolute error of a few C * 2^-24.
__device__ __forceinline__ float softcap_log2_fast(float s, float k_scaled, float C) {
  const float e = fast_exp2(s * k_scaled);
  return __builtin_fmaf(-2.0f * C, __builtin_amdgcn_rcpf(1.0f + e), C);
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Max / sum of a value across the two 32-lane halves of a wave64, broadcast
// to every lane.  v_permlane32_swap exchanges the upper 32 lanes of its first
// operand with the lower 32 lanes of its second; with two copies of v the
// operands end up holding [v.lo, v.lo] and [v.hi, v.hi].  Issued as inline
// asm on two distinct registers: the compiler builtin, given the same value
// twice, let later code treat the two halves as equal.  The s_nop covers the
// VALU-write -> permlane-read hazard.
__device__ __forceinline__ void half_swap(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float half_swap_max(float v) {
  float a = v, b = v;
  half_swap(a, b);
  return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float half_swap_sum(float v) {
  float a = v, b = v;
  half_swap(a, b);
  return a + b;
}

// Work-ordered dispatch for launches whose tiles come from BlockMask lists:
// a tile's work is its listed block count, which need not follow the tile
// index (documents).  Every wave of the launch orders the same counts and
// takes the tile at its dispatch position pos (0 <= pos < n), in the order:
// descending count (clamped to [0, cap], cap < 2^15), ties by tile index, the
// later tile first when later_first.  That is one permutation of the n
// tiles, the same in every wave.  Each wave finds its tile on its own, with
// no LDS and no barrier: the counts (n <= kOrderCap, four per lane) go into
// registers; a binary search over count values finds v, the count of the
// tile at pos (the largest v with more than pos tiles counting at least v);
// and lane prefix counts over the ballot of the tiles of count v pick the
// one at rank pos - #(count > v) among them.  With count set, v is returned
// there too, so the caller need not read the tile's count again.
constexpr int kOrderCap = 256;
__device__ inline int work_ordered_tile(const int32_t *cnt, int n, int cap, int pos, bool later_first,
                                        int *count = nullptr) {
  constexpr int KPL = kOrderCap / 64;
  const int lane = threadIdx.x & 63;
  int c[KPL];   // clamped counts of tiles lane + 64 j; -1 past n
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int t = lane + 64 * j;
    c[j] = (t < n) ? min(max(cnt[t], 0), cap) : -1;
  }
  auto count_ge = [&](int v) -> int {   // tiles whose count is at least v
    int s = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) s += __builtin_popcountll(__builtin_amdgcn_ballot_w64(c[j] >= v));
    return s;
  };
  int lo = 0, hi = cap;   // count_ge(lo) > pos holds from the start: count_ge(0) = n
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (count_ge(mid) > pos) lo = mid;
    else hi = mid - 1;
  }
  const int v = lo;
  const int k = pos - count_ge(v + 1);   // rank among the tiles of count v
  int sel = 0;
  int ahead = 0;   // tiles of count v in the lane blocks already passed
#pragma unroll
  for (int jj = 0; jj < KPL; ++jj) {
    const int j = later_first ? KPL - 1 - jj : jj;
    const bool mine = (c[j] == v);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(mine);
    const int pc = __builtin_popcountll(m);
    const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    const int r = ahead + (later_first ? pc - 1 - below : below);
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(mine && r == k);
    if (hit) sel = 64 * j + __builtin_ctzll(hit);
    ahead += pc;
  }
  if (count) *count = v;
  return sel;
}

// Stages entries [0, n) of a BlockMask list row and their flags (flags may
// be null: all 0) into LDS for a workgroup of NT threads, n <= CAP.  Every
// load (range-checked buffer loads: a slot past n reads 0) is issued before
// the first store, so the row costs one memory latency, shared with any
// loads the caller issued before; the caller's barrier publishes the row.
template <int CAP, int NT>
__device__ inline void stage_list_row(const int32_t *idx, const uint8_t *flags, int n, int32_t *s_idx,
                                      uint8_t *s_flag, int tid) {
  const __amdgpu_buffer_rsrc_t l_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)idx, (short)0, n * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t f_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(flags ? (const void *)flags : (const void *)idx), (short)0, flags ? n : 0, 0x00020000);
  constexpr int PER = CAP / NT;
  int32_t v[PER];
  uint8_t f[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (u * NT < n) {   // workgroup-uniform
      v[u] = __builtin_amdgcn_raw_buffer_load_b32(l_rsrc, (tid + u * NT) * 4, 0, 0);
      f[u] = __builtin_amdgcn_raw_buffer_load_b8(f_rsrc, tid + u * NT, 0, 0);
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int t = tid + u * NT;
    if (t < n) {
      s_idx[t] = v[u];
      s_flag[t] = f[u];
    }
  }
}

// Minimum / maximum of an int over the 64 lanes of a wave, in every lane, by
// DPP (no LDS traffic): shifts by 1, 2, 4, 8 within each 16-lane row leave
// the row's result in its lane 15; row_bcast:15 and row_bcast:31 carry it on
// to rows 1, 3 and then 2, 3, so lane 63 ends with the whole wave's result.
// Lanes a shift reads nothing for keep their own value (old = src).
template <bool MIN, int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_step(int v) {
  const int t = __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xf, false);
  return MIN ? min(v, t) : max(v, t);
}
template <bool MIN>
__device__ __forceinline__ int wave_reduce_i32(int v) {
  v = dpp_step<MIN, 0x111, 0xf>(v);   // row_shr:1
  v = dpp_step<MIN, 0x112, 0xf>(v);   // row_shr:2
  v = dpp_step<MIN, 0x114, 0xf>(v);   // row_shr:4
  v = dpp_step<MIN, 0x118, 0xf>(v);   // row_shr:8
  v = dpp_step<MIN, 0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_step<MIN, 0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_min_i32(int v) { return wave_reduce_i32<true>(v); }
__device__ __forceinline__ int wave_max_i32(int v) { return wave_reduce_i32<false>(v); }

// Round-to-nearest-even fp32 -> bf16 of two values, packed (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

}  // namespace attn
