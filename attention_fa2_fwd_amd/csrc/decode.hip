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
// kv head), so the design is about bytes in flight, not FLOPs:
//  * workgroup = (sequence, kv head, group of up to 4 query heads, split of
//    64 pages = 1024 tokens); its 4 waves take the split's pages round-robin,
//    so each K/V byte read serves every query head of the group (GQA);
//  * a page of one kv head is one contiguous 4 KiB block of K (and of V),
//    read through a buffer resource of its own (an out-of-pool page id gets
//    an empty range and reads as zeros); lane = 8 token slots x 2 chunks of
//    8 d, so each load instruction reads whole 128-byte half rows; the
//    split's page ids are read once up front and each page's id is taken
//    into a scalar register, so the loop issues no dependent loads and the
//    next page is in flight while the current one is reduced;
//  * scores use v_dot2_f32_bf16 on the packed bf16 pairs, reduced over the 8
//    slices with ds_swizzle; each lane keeps its own running max / sum / O
//    (no cross-lane traffic per token), merged across lanes and waves once
//    per split;
//  * the grid is sized from max_pages_per_seq, so the host never reads the
//    device-side lengths; splits past a sequence's end exit at once.
#include "kernels.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kSplitPages = 64;
constexpr int kD = 128;
constexpr int kPage = 16;
constexpr float kRescaleThresh = 8.0f;   // log2 units: keep p <= 2^8 between rescales
// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;

struct DecArgs {
  const __bf16 *q, *kc, *vc;
  const int32_t *page_table, *seq_lens;
  int Hq, Hkv, max_pages, num_pages, n_hgroups, max_splits;
  float scale_log2;
  ScoreArgs score;
  float *ws_o, *ws_lse;
};

__device__ __forceinline__ float swz_sum8(float v) {
  // sum over the 8 lanes of an aligned 8-lane group (xor 1, 2, 4)
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x041F));
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x081F));
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x101F));
  return v;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

template <int GH>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(DecArgs a) {
  __shared__ float red_o[4][GH][kD];
  __shared__ float red_m[4][GH];
  __shared__ float red_l[4][GH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t8 = lane >> 3;        // token slot (tokens t8 and t8 + 8 of a page)
  const int e8 = lane & 7;         // d chunks [8 e8, 8 e8 + 8) and [64 + 8 e8, 64 + 8 e8 + 8)
  const int split = blockIdx.x;
  const int hkv = blockIdx.y / a.n_hgroups;
  const int hg = blockIdx.y - hkv * a.n_hgroups;
  const int s = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int hq0 = hkv * G + hg * GH;

  const int L = a.seq_lens[s];
  const int n_pages = min(a.max_pages, (max(L, 0) + kPage - 1) / kPage);
  const int p_begin = split * kSplitPages;
  if (p_begin >= n_pages) return;                      // uniform across the workgroup
  const int p_end = min(n_pages, p_begin + kSplitPages);
  const int qpos = L - 1;

  // Page ids of the split, one per lane (kSplitPages == 64), read once so the
  // page loop issues no dependent loads: each page's id is taken with
  // readlane into a scalar register.
  static_assert(kSplitPages == 64, "one page id per lane");
  const int32_t *ptab = a.page_table + (size_t)s * a.max_pages;
  const int my_page = (p_begin + lane < p_end) ? ptab[p_begin + lane] : -1;

  // This lane's slice of the GH queries, as packed bf16 pairs (the same two
  // d chunks as its K/V loads).
  uint32_t qv[GH][8];
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    const __bf16 *src = a.q + ((size_t)s * a.Hq + hq0 + g) * kD;
    const u32x4 w0 = *(const u32x4 *)(src + 8 * e8);
    const u32x4 w1 = *(const u32x4 *)(src + 64 + 8 * e8);
    qv[g][0] = w0[0]; qv[g][1] = w0[1]; qv[g][2] = w0[2]; qv[g][3] = w0[3];
    qv[g][4] = w1[0]; qv[g][5] = w1[1]; qv[g][6] = w1[2]; qv[g][7] = w1[3];
  }
  float bias2[GH];
#pragma unroll
  for (int g = 0; g < GH; ++g) bias2[g] = bias_coeff(a.score, hq0 + g, a.Hq) * kLog2e;
  const bool has_bias = a.score.kind != ATTN_SCORE_NONE;

  float m[GH], l[GH], o[GH][16];
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int d = 0; d < 16; ++d) o[g][d] = 0.0f;
  }

  // One (page, kv head) block is 16 tokens x 256 bytes of K (and of V).  A
  // buffer resource per block: an id outside the pool gets an empty range,
  // so its loads return zeros without any wait or branch.
  constexpr int kBlockBytes = kPage * kD * 2;
  auto block_rsrc = [&](const __bf16 *cache, int page) {
    const bool ok = (page >= 0) && (page < a.num_pages);
    const __bf16 *base = cache + ((size_t)(ok ? page : 0) * a.Hkv + hkv) * (kPage * kD);
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, ok ? kBlockBytes : 0, kBufferFlags);
  };
  // Lane (t8, e8) loads 16 bytes at d 8 e8 and 16 at d 64 + 8 e8 of tokens
  // t8 and t8 + 8: each load instruction reads 8 whole 128-byte half rows.
  const int ld_off = t8 * (kD * 2) + e8 * 16;
  // Loads are issued for every prefetch slot, past the split's end too (as
  // an empty range), so the number of loads in flight is the same on every
  // path and each wait covers only the page about to be reduced.
  auto load_page = [&](int pi, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
    const int page = (pi < p_end) ? __builtin_amdgcn_readlane(my_page, min(pi - p_begin, 63)) : -1;
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.kc, page);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.vc, page);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int off = ld_off + (i & 1) * 128 + (i >> 1) * 8 * (kD * 2);
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  };

  auto process_page = [&](int pi, const u32x4 (&kr)[4], const u32x4 (&vr)[4]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int j = pi * kPage + t8 + 8 * tt;
      const bool valid = j < L;
      float x[GH];
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t kw = kr[2 * tt + (u >> 2)][u & 3];
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv[g][u]),
                                                __builtin_bit_cast(bf16x2, kw), acc, false);
        }
        acc = swz_sum8(acc);
        float xx = acc * a.scale_log2;
        if (has_bias) xx += bias2[g] * (float)(j - qpos);
        x[g] = valid ? xx : -INFINITY;
      }
      // Rescale only when a score exceeds the running max by the threshold
      // (the max is a stabiliser; the result does not depend on its value).
#pragma unroll
      for (int g = 0; g < GH; ++g) {
        if (x[g] > m[g] + kRescaleThresh) {
          const float alpha = fast_exp2(m[g] - x[g]);   // 0 when m = -inf
          l[g] *= alpha;
#pragma unroll
          for (int d = 0; d < 16; ++d) o[g][d] *= alpha;
          m[g] = x[g];
        }
      }
      float vf[16];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t vw = vr[2 * tt + (u >> 2)][u & 3];
        vf[2 * u] = bf_lo(vw);
        vf[2 * u + 1] = bf_hi(vw);
      }
      // Tokens past the sequence end (tail of the last page) are skipped,
      // not weighted by 0, so whatever those slots hold cannot leak in.
      if (valid) {
#pragma unroll
        for (int g = 0; g < GH; ++g) {
          const float p = fast_exp2(x[g] - m[g]);
          l[g] += p;
#pragma unroll
          for (int d = 0; d < 16; ++d) o[g][d] = fmaf(p, vf[d], o[g][d]);
        }
      }
    }
  };

  // Pages of this split, round-robin over the waves, next page prefetched.
  int pi = p_begin + wave;
  u32x4 ka[4], va[4], kb[4], vb[4];
  load_page(pi, ka, va);
  while (pi < p_end) {
    load_page(pi + 4, kb, vb);
    process_page(pi, ka, va);
    pi += 4;
    if (pi >= p_end) break;
    load_page(pi + 4, ka, va);
    process_page(pi, kb, vb);
    pi += 4;
  }

  // Merge the 8 token slots of the wave (lanes e8, e8 + 8, ..., e8 + 56).
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    float mm = m[g];
    mm = fmaxf(mm, __shfl_xor(mm, 8));
    mm = fmaxf(mm, __shfl_xor(mm, 16));
    mm = fmaxf(mm, __shfl_xor(mm, 32));
    const float f = (m[g] == -INFINITY) ? 0.0f : fast_exp2(m[g] - mm);
    float lg = l[g] * f;
    lg += __shfl_xor(lg, 8);
    lg += __shfl_xor(lg, 16);
    lg += __shfl_xor(lg, 32);
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      float v = o[g][d] * f;
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[g][d] = v;
    }
    if (lane < 8) {
#pragma unroll
      for (int d = 0; d < 16; ++d) red_o[wave][g][(d < 8 ? 0 : 56) + 8 * e8 + d] = o[g][d];
      if (lane == 0) {
        red_m[wave][g] = mm;
        red_l[wave][g] = lg;
      }
    }
  }
  __syncthreads();

  // Merge the 4 waves; write the normalised partial and its natural-log LSE.
  for (int idx = tid; idx < GH * kD; idx += kThreads) {
    const int g = idx / kD;
    const int d = idx - g * kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][g]);
    float acc = 0.0f, tot = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (red_m[w][g] == -INFINITY) ? 0.0f : fast_exp2(red_m[w][g] - M);
      acc = fmaf(red_o[w][g][d], f, acc);
      tot = fmaf(red_l[w][g], f, tot);
    }
    const size_t row = ((size_t)s * a.Hq + hq0 + g) * a.max_splits + split;
    a.ws_o[row * kD + d] = acc / tot;
    if (d == 0) a.ws_lse[row] = (M + fast_log2(tot)) * kLn2;
  }
}

struct CombArgs {
  const int32_t *seq_lens;
  int Hq, max_pages, max_splits;
  const float *ws_o, *ws_lse;
  __bf16 *out;
  float *lse;
};

// One workgroup per (sequence, query head); thread d owns output column d.
__global__ __launch_bounds__(kD) void decode_combine_kernel(CombArgs a) {
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  const int L = a.seq_lens[s];
  const int n_pages = min(a.max_pages, (max(L, 0) + kPage - 1) / kPage);
  const int ns = (n_pages + kSplitPages - 1) / kSplitPages;
  const size_t row0 = ((size_t)s * a.Hq + hq) * a.max_splits;
  float M = -INFINITY;
  for (int k = 0; k < ns; ++k) M = fmaxf(M, a.ws_lse[row0 + k]);
  float acc = 0.0f, tot = 0.0f;
  for (int k = 0; k < ns; ++k) {
    const float w = fast_exp2((a.ws_lse[row0 + k] - M) * kLog2e);
    tot += w;
    acc = fmaf(w, a.ws_o[(row0 + k) * kD + d], acc);
  }
  const size_t orow = (size_t)s * a.Hq + hq;
  a.out[orow * kD + d] = (__bf16)((tot > 0.0f) ? acc / tot : 0.0f);
  if (d == 0) a.lse[orow] = (tot > 0.0f) ? M + logf(tot) : -INFINITY;
}

}  // namespace

void decode_split_geometry(int max_pages, int *split_pages, int *max_splits) {
  *split_pages = kSplitPages;
  *max_splits = (max_pages + kSplitPages - 1) / kSplitPages;
}

hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const int GH = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  DecArgs a;
  a.q = (const __bf16 *)p.q;
  a.kc = (const __bf16 *)p.k_cache;
  a.vc = (const __bf16 *)p.v_cache;
  a.page_table = p.page_table;
  a.seq_lens = p.seq_lens;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.max_pages = p.max_pages;
  a.num_pages = p.num_pages;
  a.n_hgroups = G / GH;
  a.max_splits = p.max_splits;
  a.scale_log2 = p.scale * kLog2e;
  a.score = p.score;
  a.ws_o = p.ws_o;
  a.ws_lse = p.ws_lse;
  const dim3 grid(p.max_splits, p.Hkv * a.n_hgroups, p.N);
  if (GH == 4) hipLaunchKernelGGL(decode_split_kernel<4>, grid, dim3(kThreads), 0, stream, a);
  else if (GH == 2) hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CombArgs c;
  c.seq_lens = p.seq_lens;
  c.Hq = p.Hq;
  c.max_pages = p.max_pages;
  c.max_splits = p.max_splits;
  c.ws_o = p.ws_o;
  c.ws_lse = p.ws_lse;
  c.out = (__bf16 *)p.out;
  c.lse = p.lse;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(p.Hq, p.N), dim3(kD), 0, stream, c);
  return hipGetLastError();
}

}  // namespace attn
