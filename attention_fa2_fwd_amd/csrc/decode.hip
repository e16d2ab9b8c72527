// Paged split-KV decode: one query per sequence against its paged K/V cache,
// split along the keys, each split reduced with an online softmax, then the
// splits merged by log-sum-exp.  PagedAttention is named in the FlexAttention
// write-up's variant list; a multi-query paged-attention kernel is described
// in "高级特性：探索PyTorch/XLA的Pallas内核和Flash Attention实现".  The merge
// is the online-softmax rescaling of "Attention优化｜2w字原理&图解: 从
// Online-Softmax到FlashAttention V1/V2/V3" (abstract) applied to whole
// partial results: LSE = ln sum_k e^{lse_k}, O = sum_k e^{lse_k - LSE} O_k.
//
// The work is bound by HBM bandwidth (every valid K/V byte is read once per
// kv head), so the design keeps many bytes in flight and the arithmetic off
// the critical path:
//  * workgroup = (kv head, work item), the items being the splits of every
//    sequence in order (64 pages, 1024 tokens, each; 32 or 16 when that
//    leaves too few items to fill the chip).  When every key range fits 128
//    pages (short caches, windows up to 2032 keys) and the sequences x kv
//    heads give at least 256 items, each sequence is one item, reduced
//    straight into the output: no partials and no merge launch (a 1024-key
//    window: 51.8 -> 45.5 us per call on the 64-sequence workload).  A
//    workgroup finds its
//    (sequence, split) from a prefix sum of the sequences' split counts, so
//    the dispatch order holds every live item first and the workgroups past
//    the last item (the grid is sized from max_pages_per_seq and the window,
//    as the host never reads the device-side lengths) come last and exit at
//    once.  The
//    4 waves take the split's pages round-robin.  All G <= 16 query heads of
//    the kv head are processed together, so each K/V byte read serves every
//    query head of the group (GQA);
//  * the arithmetic is on the matrix cores: per page, S^T = K Q^T is four
//    v_mfma_f32_16x16x32_bf16 (16 tokens x 16 head columns) and O^T += V^T P^T
//    eight v_mfma_f32_16x16x16_bf16; the S^T accumulator is already the B
//    operand of the second product, and V^T comes from ds_read_b64_tr_b16;
//  * a page of one kv head is one contiguous 4 KiB block of K (and of V),
//    read through a buffer resource of its own whose range ends at the
//    sequence's last token: slots past it and out-of-pool page ids read as
//    zeros, so they can never inject NaN through a zero weight.  K goes to
//    registers (already in the MFMA A layout); V goes to LDS through
//    buffer_load ... lds, three pages per wave in flight, into three LDS
//    objects named at every access so that each read waits only for its
//    own page;
//  * the split's page ids are read once up front and each page's id is taken
//    into a scalar register, so the page loop issues no dependent loads.
#include "kernels.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxSplitPages = 64;   // one page id per lane
// A key range of at most this many pages is one work item per (sequence, kv
// head), reduced straight into the output: no partials, no merge launch.
constexpr int kDirectPages = 128;    // two page ids per lane
// ... when that still gives at least one workgroup per compute unit.
constexpr long kDirectMinItems = 256;
constexpr int kMinSplitPages = 16;   // four pages per wave
// Items wanted in the grid before the splits are made smaller: about eight
// workgroups per compute unit.
constexpr long kTargetItems = 2048;
constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kRowBytes = kD * 2;
constexpr int kBlockBytes = kPage * kRowBytes;   // one (page, kv head) block of K or V
constexpr float kRescaleThresh = 8.0f;           // log2 units: keep p <= 2^8 between rescales
// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;
// Cache policy bits of the K/V loads: the default (measured faster here than
// the non-temporal hint, although every byte is read once).
constexpr int kStreamAux = 0;

typedef __attribute__((address_space(3))) void lds_void;

// Keys a decode query sees: t in [t0, L) with t0 = max(0, L - window) under a
// sliding window (window = 0: no window), held in pages [pf, pe).
__device__ __forceinline__ void key_range(int L, int window, int max_pages, int &t0, int &pf, int &pe) {
  L = max(L, 0);
  pe = min(max_pages, (L + kPage - 1) / kPage);
  t0 = window > 0 ? max(0, L - window) : 0;
  pf = min(t0 / kPage, pe);
}

struct DecArgs {
  const __bf16 *q, *kc, *vc;
  const int32_t *page_table, *seq_lens;
  int n_seq, Hq, Hkv, max_pages, num_pages, max_splits;
  int split_pages; // pages per split, kMinSplitPages .. kMaxSplitPages
  int window;      // sliding window of the decode query, 0 = none
  int direct;      // 1: one item per (sequence, kv head) of up to kDirectPages pages, written to out / lse
  float scale_log2;
  ScoreArgs score;
  float *ws_o, *ws_lse;
  __bf16 *out;
  float *lse;
};

__device__ __forceinline__ s16x4 lds_read_tr(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}

// Three workgroups per CU (168 VGPRs, 48 KiB of LDS each) keep more pages
// in flight than two: measured 0.6% faster unwindowed and 6% with a window.
__global__ __launch_bounds__(kThreads, 3) void decode_split_kernel(DecArgs a) {
  // V pages staged per wave: three slots, three separate LDS objects.
  __shared__ __align__(16) char v_lds0[kWaves][kBlockBytes];
  __shared__ __align__(16) char v_lds1[kWaves][kBlockBytes];
  __shared__ __align__(16) char v_lds2[kWaves][kBlockBytes];
  __shared__ float red_m[kWaves][16];
  __shared__ float red_l[kWaves][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;     // MFMA column: query head hq0 + col
  const int grp = lane >> 4;     // 16-lane group
  const int hkv = blockIdx.x % a.Hkv;

  // Work item blockIdx.x / Hkv: the items are the splits of sequence 0, then
  // of sequence 1, ...  Find (s, split) from the inclusive prefix sum of the
  // split counts, 64 sequences at a time.
  int s = -1, split = 0;
  {
    int w = blockIdx.x / a.Hkv;
    for (int c0 = 0; c0 < a.n_seq && s < 0; c0 += 64) {
      const int i = c0 + lane;
      int ns = 0;
      if (i < a.n_seq) {
        int t0, pf, pe;
        key_range(a.seq_lens[i], a.window, a.max_pages, t0, pf, pe);
        ns = a.direct ? 1 : (pe - pf + a.split_pages - 1) / a.split_pages;
      }
      int incl = ns;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const unsigned long long hit = __ballot(incl > w);
      if (hit) {
        const int f = __builtin_ctzll(hit);
        s = c0 + f;
        split = w - (__shfl(incl, f) - __shfl(ns, f));
      } else {
        w -= __shfl(incl, 63);
      }
    }
    s = __builtin_amdgcn_readfirstlane(s);
    split = __builtin_amdgcn_readfirstlane(split);
  }
  if (s < 0) return;                                   // past the last item (uniform)
  const int G = a.Hq / a.Hkv;
  const int hq0 = hkv * G;

  // The length is uniform; taken into a scalar register, everything derived
  // from it (page range, buffer ranges) stays scalar.
  const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[s]);
  int t0, p_first, p_stop;
  key_range(L, a.window, a.max_pages, t0, p_first, p_stop);
  t0 = __builtin_amdgcn_readfirstlane(t0);
  const int p_begin = __builtin_amdgcn_readfirstlane(p_first + split * a.split_pages);
  const int p_end = __builtin_amdgcn_readfirstlane(min(p_stop, p_begin + (a.direct ? kDirectPages : a.split_pages)));
  const int qpos = L - 1;

  // Page ids of the split, one per lane (two for a direct item), read once.
  static_assert(kMaxSplitPages <= 64 && kDirectPages <= 128, "page ids per lane");
  const int32_t *ptab = a.page_table + (size_t)s * a.max_pages;
  const int my_page = (p_begin + lane < p_end) ? ptab[p_begin + lane] : -1;
  const int my_page2 = (p_begin + 64 + lane < p_end) ? ptab[p_begin + 64 + lane] : -1;

  // Q^T fragments, the B operand of S^T = K Q^T: lane holds
  // Q[hq0 + col][32c + 8 grp .. + 7]; columns past the group are zero.
  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qf[c] = bf16x8{};
    if (col < G) qf[c] = *(const bf16x8 *)(a.q + ((size_t)s * a.Hq + hq0 + col) * kD + 32 * c + 8 * grp);
  }
  const float bias2 = (col < G) ? bias_coeff(a.score, hq0 + col, a.Hq) * kLog2e : 0.0f;
  const bool has_bias = a.score.kind == ATTN_SCORE_ALIBI || a.score.kind == ATTN_SCORE_REL_POS;
  const bool has_cap = a.score.kind == ATTN_SCORE_SOFTCAP;
  const float cap2 = has_cap ? a.score.softcap * kLog2e : 0.0f;
  const float cap_k = has_cap ? 2.0f / a.score.softcap : 0.0f;

  // O^T accumulators: o[blk][i] = O[head col][d = 16 blk + 4 grp + i].
  f32x4 o[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) o[b] = f32x4{};
  float m_run = -INFINITY;   // reference max of column col (same in all 4 groups)
  float l_run = 0.0f;        // this lane's share of the column's sum

  // Buffer resource of one (page, kv head) block, its range cut at the
  // sequence's last token.
  auto block_rsrc = [&](const __bf16 *cache, int page, int valid_bytes) __attribute__((always_inline)) {
    const bool ok = (page >= 0) && (page < a.num_pages);
    const __bf16 *base = cache + ((size_t)(ok ? page : 0) * a.Hkv + hkv) * (kPage * kD);
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, ok ? valid_bytes : 0, kBufferFlags);
  };
  // K fragment c of a page (A operand): lane holds K[token col][32c + 8 grp .. + 7].
  const int k_off = col * kRowBytes + 16 * grp;
  // V staging: load i writes rows 4i .. 4i + 3 of the block, lane L at byte
  // 1024 i + 16 L (row 4i + L/16, slot L%16), taking the row's 16-byte chunk
  // (L%16) ^ 2(L/16).  Row t of the staged block thus holds chunk c at slot
  // c ^ 2(t%4), which spreads the transposed reads below over distinct banks.
  const int v_off = (lane >> 4) * kRowBytes + 16 * ((lane & 15) ^ (2 * (lane >> 4)));
  // Transposed V reads (A operand of O^T += V^T P^T, 16 d x 16 tokens): lane
  // (grp, col) points at row t = 4 grp + col/4, d = 16 blk + 4 (col%4), i.e.
  // chunk 2 blk + (col%4)/2 at slot 2 (blk ^ (col/4)) + (col%4)/2.  For
  // blk = 4 b1 + b0 that is v_rd[b0] + 128 b1.
  const int y = col >> 2;
  int v_rd[4];
#pragma unroll
  for (int b0 = 0; b0 < 4; ++b0) v_rd[b0] = (4 * grp + y) * kRowBytes + 32 * (b0 ^ y) + 8 * (col & 3);

  // Issue the loads of page pi: K fragments into kf, V into the LDS slot vt.
  // Past the split's end the range is empty (the loads still issue, so the
  // number in flight is the same on every path).
  auto issue_page = [&](int pi, bf16x8 (&kf)[4], char *vt) __attribute__((always_inline)) {
    const int idx = pi - p_begin;
    const int page = (pi >= p_end) ? -1
                     : (idx < 64) ? __builtin_amdgcn_readlane(my_page, idx)
                                  : __builtin_amdgcn_readlane(my_page2, min(idx - 64, 63));
    // Bytes of the block before the sequence's end (scalar: written with
    // selects, not a min/max clamp that may be placed on the VALU).
    const int rem = L - pi * kPage;
    const int valid = rem >= kPage ? kBlockBytes : (rem > 0 ? rem * kRowBytes : 0);
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.kc, page, valid);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.vc, page, valid);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + 64 * c, 0, kStreamAux));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(vt + 1024 * i), 16, v_off + 1024 * i, 0, 0,
                                               kStreamAux);
  };

  // Online softmax and P.V of page pi.
  auto process = [&](int pi, const bf16x8 (&kf)[4], const char *vt) __attribute__((always_inline)) {
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int c = 0; c < 4; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[c], sacc, 0, 0, 0);
    // sacc[i]: score of token 4 grp + i for head col.
    const int j0 = pi * kPage + 4 * grp;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = sacc[i] * a.scale_log2;
      if (has_bias) v = __builtin_fmaf(bias2, (float)(j0 + i - qpos), v);
      if (has_cap) v = softcap_log2_fast(v, cap_k, cap2);
      x[i] = (j0 + i < L && j0 + i >= t0) ? v : -INFINITY;
    }
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // Raise the reference max only past the threshold.
    const bool need = tmax > m_run + kRescaleThresh;
    if (__any(need)) {
      const float m_new = need ? tmax : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;   // 0 when m_run = -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < 8; ++b) o[b] *= alpha;
    }
    const float mu = (m_run == -INFINITY) ? 0.0f : m_run;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - mu);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    // P^T (B operand, 16 tokens x 16 heads): lane holds P[token 4 grp + j][col].
    const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
    // The V^T fragment of a lane covers the same tokens 4 grp + j as its P^T
    // fragment.  In the page that holds the window's first key, the rows of
    // the keys before it are cleared: their p is 0, but 0 times a NaN left in
    // the cache is not 0.  The test is uniform, so other pages skip it.
    if (pi * kPage < t0) {
      uint64_t keep = ~0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j0 + j < t0) keep &= ~(0xffffull << (16 * j));
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t raw = __builtin_bit_cast(uint64_t, lds_read_tr(vt + v_rd[b & 3] + 128 * (b >> 2)));
        const s16x4 va = __builtin_bit_cast(s16x4, raw & keep);
        o[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[b], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const s16x4 va = lds_read_tr(vt + v_rd[b & 3] + 128 * (b >> 2));
        o[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[b], 0, 0, 0);
      }
    }
  };

  // Pages of this split, round-robin over the waves, two pages ahead.
  int pi = p_begin + wave;
  bf16x8 k0[4], k1[4], k2[4];
  issue_page(pi, k0, v_lds0[wave]);
  issue_page(pi + kWaves, k1, v_lds1[wave]);
  while (pi < p_end) {
    issue_page(pi + 2 * kWaves, k2, v_lds2[wave]);
    process(pi, k0, v_lds0[wave]);
    pi += kWaves;
    if (pi >= p_end) break;
    issue_page(pi + 2 * kWaves, k0, v_lds0[wave]);
    process(pi, k1, v_lds1[wave]);
    pi += kWaves;
    if (pi >= p_end) break;
    issue_page(pi + 2 * kWaves, k1, v_lds1[wave]);
    process(pi, k2, v_lds2[wave]);
    pi += kWaves;
  }

  // Merge the waves.  Every staging load has landed before the V slots are
  // reused for the partial O of each wave: [wave][head][d] as floats.
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  static_assert(kWaves * 16 * kD * 4 <= 2 * kWaves * kBlockBytes, "partials fit in two V slots");
  float *red_o0 = (float *)&v_lds0[0][0];   // waves 0, 1
  float *red_o1 = (float *)&v_lds1[0][0];   // waves 2, 3
  float *mine = (wave < 2 ? red_o0 : red_o1) + (wave & 1) * 16 * kD;
  if (col < G) {
#pragma unroll
    for (int b = 0; b < 8; ++b)
      *(f32x4 *)(mine + col * kD + 16 * b + 4 * grp) = o[b];
    if (grp == 0) {
      red_m[wave][col] = m_run;
      red_l[wave][col] = lt;
    }
  }
  __syncthreads();

  // Normalised partial and its natural-log LSE per (head, split).
  for (int idx = tid; idx < G * kD; idx += kThreads) {
    const int g = idx / kD;
    const int d = idx - g * kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][g]);
    float acc = 0.0f, tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = (red_m[w][g] == -INFINITY) ? 0.0f : fast_exp2(red_m[w][g] - M);
      const float *ow = (w < 2 ? red_o0 : red_o1) + (w & 1) * 16 * kD;
      acc = fmaf(ow[g * kD + d], f, acc);
      tot = fmaf(red_l[w][g], f, tot);
    }
    if (a.direct) {
      // The item is the whole key range: its normalised O and LSE are the
      // output (no visible key: O = 0, LSE = -inf, as the merge writes them).
      const size_t item = (size_t)s * a.Hq + hq0 + g;
      a.out[item * kD + d] = (__bf16)((tot > 0.0f) ? acc / tot : 0.0f);
      if (d == 0) a.lse[item] = (tot > 0.0f) ? (M + fast_log2(tot)) * kLn2 : -INFINITY;
    } else {
      const size_t row = ((size_t)s * a.Hq + hq0 + g) * a.max_splits + split;
      a.ws_o[row * kD + d] = acc / tot;
      if (d == 0) a.ws_lse[row] = (M + fast_log2(tot)) * kLn2;
    }
  }
}

struct CombArgs {
  const int32_t *seq_lens;
  int n_items;   // N * Hq
  int Hq, max_pages, max_splits, split_pages, window;
  const float *ws_o, *ws_lse;
  __bf16 *out;
  float *lse;
};

// One wave per (sequence, query head).  The lanes take the splits' LSEs, 64
// at a time, for the reference max M and the weight sum; lane l then owns
// output columns 2l and 2l + 1 and accumulates the splits' partials with the
// weights e^(lse_k - M), taken per split from the lane that holds them.
constexpr int kCombWaves = 4;
__global__ __launch_bounds__(64 * kCombWaves) void decode_combine_kernel(CombArgs a) {
  static_assert(kD == 128, "two output columns per lane");
  const int lane = threadIdx.x & 63;
  const int item = (int)blockIdx.x * kCombWaves + (int)(threadIdx.x >> 6);   // s * Hq + hq
  if (item >= a.n_items) return;                                            // uniform per wave
  const int s = item / a.Hq;
  int t0, pf, pe;
  key_range(a.seq_lens[s], a.window, a.max_pages, t0, pf, pe);
  const int ns = __builtin_amdgcn_readfirstlane((pe - pf + a.split_pages - 1) / a.split_pages);
  const size_t row0 = (size_t)item * a.max_splits;
  float M = -INFINITY;
  for (int k0 = 0; k0 < ns; k0 += 64)
    if (k0 + lane < ns) M = fmaxf(M, a.ws_lse[row0 + k0 + lane]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc0 = 0.0f, acc1 = 0.0f, tot = 0.0f;
  const f32x2 *po = (const f32x2 *)(a.ws_o + row0 * kD) + lane;
  for (int k0 = 0; k0 < ns; k0 += 64) {
    const float wl = (k0 + lane < ns) ? fast_exp2((a.ws_lse[row0 + k0 + lane] - M) * kLog2e) : 0.0f;
    tot += wl;
    const int kn = min(64, ns - k0);
    auto take = [&](int j, f32x2 v) __attribute__((always_inline)) {
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), j));
      acc0 = fmaf(w, v[0], acc0);
      acc1 = fmaf(w, v[1], acc1);
    };
    int j = 0;
    for (; j + 16 <= kn; j += 16) {   // sixteen independent row loads in flight
      f32x2 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = po[(size_t)(k0 + j + u) * (kD / 2)];
#pragma unroll
      for (int u = 0; u < 16; ++u) take(j + u, v[u]);
    }
    for (; j + 4 <= kn; j += 4) {
      f32x2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = po[(size_t)(k0 + j + u) * (kD / 2)];
#pragma unroll
      for (int u = 0; u < 4; ++u) take(j + u, v[u]);
    }
    for (; j < kn; ++j) take(j, po[(size_t)(k0 + j) * (kD / 2)]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
  const float inv = (tot > 0.0f) ? 1.0f / tot : 0.0f;
  *(uint32_t *)(a.out + (size_t)item * kD + 2 * lane) = pack_bf16x2(acc0 * inv, acc1 * inv);
  if (lane == 0) a.lse[item] = (tot > 0.0f) ? M + logf(tot) : -INFINITY;
}

}  // namespace

int decode_max_splits(int max_pages) { return (max_pages + kMinSplitPages - 1) / kMinSplitPages; }

namespace {
// Pages a sequence's key range may span: all of max_pages, or under a window
// of W keys at most (W - 1) / page + 2 (the window need not start on a page
// boundary).
int pages_bound(int max_pages, int window) {
  if (window <= 0) return max_pages;
  return (int)std::min<long>(max_pages, (long)(window - 1) / kPage + 2);
}
// The largest split size that still gives kTargetItems items, assuming every
// sequence is as long as the bound.
int choose_split_pages(int n_seq, int Hkv, int bound) {
  for (int sp = kMaxSplitPages; sp > kMinSplitPages; sp /= 2)
    if ((long)n_seq * Hkv * ((bound + sp - 1) / sp) >= kTargetItems) return sp;
  return kMinSplitPages;
}
}  // namespace

namespace {
// Direct items when every key range fits one and there are enough of them.
bool use_direct(int n_seq, int Hkv, int bound) {
  return bound <= kDirectPages && (long)n_seq * Hkv >= kDirectMinItems;
}
}  // namespace

int decode_launch_splits(const DecodeParams &p) {
  const int window = (p.mask.kind == ATTN_MASK_SLIDING) ? p.mask.window : 0;
  const int bound = pages_bound(p.max_pages, window);
  if (use_direct(p.N, p.Hkv, bound)) return 0;   // no workspace used
  const int sp = choose_split_pages(p.N, p.Hkv, bound);
  return (bound + sp - 1) / sp;
}

hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream) {
  DecArgs a;
  a.n_seq = p.N;
  a.window = (p.mask.kind == ATTN_MASK_SLIDING) ? p.mask.window : 0;
  a.q = (const __bf16 *)p.q;
  a.kc = (const __bf16 *)p.k_cache;
  a.vc = (const __bf16 *)p.v_cache;
  a.page_table = p.page_table;
  a.seq_lens = p.seq_lens;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.max_pages = p.max_pages;
  a.num_pages = p.num_pages;
  a.max_splits = p.max_splits;
  const int bound = pages_bound(p.max_pages, a.window);
  a.direct = use_direct(p.N, p.Hkv, bound) ? 1 : 0;
  a.split_pages = choose_split_pages(p.N, p.Hkv, bound);
  a.scale_log2 = p.scale * kLog2e;
  a.score = p.score;
  a.ws_o = p.ws_o;
  a.ws_lse = p.ws_lse;
  a.out = (__bf16 *)p.out;
  a.lse = p.lse;
  // Items that can be live: splits of the longest possible key range (one
  // per sequence for direct items).
  const int splits = a.direct ? 1 : (bound + a.split_pages - 1) / a.split_pages;
  if (!a.direct && splits > p.max_splits) return hipErrorInvalidValue;
  const size_t n_wg = (size_t)p.N * splits * p.Hkv;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_wg);
  hipLaunchKernelGGL(decode_split_kernel, grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.direct) return e;
  CombArgs c;
  c.seq_lens = p.seq_lens;
  c.n_items = p.N * p.Hq;
  c.Hq = p.Hq;
  c.max_pages = p.max_pages;
  c.max_splits = p.max_splits;
  c.split_pages = a.split_pages;
  c.window = a.window;
  c.ws_o = p.ws_o;
  c.ws_lse = p.ws_lse;
  c.out = (__bf16 *)p.out;
  c.lse = p.lse;
  const unsigned comb_grid = (unsigned)((c.n_items + kCombWaves - 1) / kCombWaves);
  hipLaunchKernelGGL(decode_combine_kernel, dim3(comb_grid), dim3(64 * kCombWaves), 0, stream, c);
  return hipGetLastError();
}

}  // namespace attn
