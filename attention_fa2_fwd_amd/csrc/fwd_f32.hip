// Fused attention forward, fp32 inputs and arithmetic (VALU FMA; no MFMA).
//
// Same result as the bf16 path — softmax(score_mod(scale·Q·Kᵀ) masked)·V with
// the log-sum-exp, FlexAttention write-up §FlexAttention — in the 1-pass
// online-softmax form ("Attention优化｜2w字原理&图解: 从Online-Softmax到
// FlashAttention V1/V2/V3", abstract), kept in fp32 end to end for inputs that
// need fp32 accuracy.  A workgroup owns 64 query rows; four lanes share a row
// (each holds a quarter of its d range), and 32-key K/V tiles (16 at D = 256)
// are staged through LDS.
#include "kernels.h"

namespace attn {
namespace {

constexpr int kRows = 64;
constexpr int kThreads = 256;

struct F32Args {
  const float *q, *k, *v;
  float *out, *lse;
  int B, Hq, Hkv, Sq, Skv, n_qtiles;
  float scale_log2;
  MaskArgs mask;
  ScoreArgs score;
  const int32_t *bm_num, *bm_idx;
  int bm_nqb, bm_nkb, bm_batch, bm_kv_block;
};

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args a) {
  constexpr int TK = (D >= 256) ? 16 : 32;   // keys per LDS tile
  constexpr int DQ = D / 4;                  // d values per lane
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];

  const int tid = threadIdx.x;
  const int quarter = tid & 3;
  const int bh_count = a.B * a.Hq;
  const int qt = a.n_qtiles - 1 - (int)(blockIdx.x / bh_count);
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hkv = (hq * a.Hkv) / a.Hq;
  const int q0 = qt * kRows;
  const int qi = q0 + (tid >> 2);
  const bool row_ok = qi < a.Sq;

  const size_t q_base = ((size_t)(b * a.Hq + hq) * a.Sq) * D;
  const size_t kv_base = ((size_t)(b * a.Hkv + hkv) * a.Skv) * D;

  float qv[DQ], acc[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    qv[e] = row_ok ? a.q[q_base + (size_t)qi * D + quarter * DQ + e] : 0.0f;
    acc[e] = 0.0f;
  }
  float m_run = -INFINITY, l_run = 0.0f;

  const int mk = a.mask.kind;
  const float bias2 = bias_coeff(a.score, hq, a.Hq) * kLog2e;
  const bool has_bias = a.score.kind == ATTN_SCORE_ALIBI || a.score.kind == ATTN_SCORE_REL_POS;
  const bool has_cap = a.score.kind == ATTN_SCORE_SOFTCAP;
  const float cap2 = a.score.softcap * kLog2e;   // the cap in log2 units
  const bool has_doc = mk == ATTN_MASK_DOCUMENT || mk == kMaskDocWindow;
  const int32_t *doc_row = has_doc ? a.mask.doc_ids + (size_t)b * a.mask.doc_stride
                                                      : nullptr;
  const int doc_i = (doc_row && row_ok) ? doc_row[qi] : -1;

  // Key ranges: the listed blocks of the BlockMask, or one analytic range.
  const int qlast = min(q0 + kRows, a.Sq) - 1;
  int n_ranges = 1;
  int lo0 = 0, hi0 = a.Skv;
  const int32_t *list = nullptr;
  if (a.bm_num) {
    const int bb = (a.bm_batch == 1) ? 0 : b;
    const size_t row = (size_t)bb * a.bm_nqb + (q0 / 128);
    n_ranges = min(max(a.bm_num[row], 0), a.bm_nkb);
    list = a.bm_idx + row * a.bm_nkb;
  } else if (mk == ATTN_MASK_CAUSAL || mk == ATTN_MASK_DOCUMENT) {
    hi0 = min(a.Skv, qlast + 1);
  } else if (mk == ATTN_MASK_SLIDING || mk == kMaskDocWindow) {
    hi0 = min(a.Skv, qlast + 1);
    lo0 = max(0, q0 - a.mask.window + 1);
  } else if (mk == ATTN_MASK_PREFIX_LM) {
    hi0 = min(a.Skv, max(qlast + 1, a.mask.prefix_len));
  }

  for (int rgi = 0; rgi < n_ranges; ++rgi) {
    int lo = lo0, hi = hi0;
    if (list) {
      const int blk = list[rgi];
      if (blk < 0 || blk >= a.bm_nkb) continue;
      lo = blk * a.bm_kv_block;
      hi = min(a.Skv, lo + a.bm_kv_block);
    }
    for (int t0 = lo; t0 < hi; t0 += TK) {
      __syncthreads();
      for (int c = tid; c < TK * D; c += kThreads) {
        const int r = c / D, col = c % D;
        const int key = t0 + r;
        const bool ok = key < hi;
        ks[r][col] = ok ? a.k[kv_base + (size_t)key * D + col] : 0.0f;
        vs[r][col] = ok ? a.v[kv_base + (size_t)key * D + col] : 0.0f;
      }
      __syncthreads();
      const int nk = min(TK, hi - t0);
      for (int jj = 0; jj < nk; ++jj) {
        const int j = t0 + jj;
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < DQ; ++e) part = fmaf(qv[e], ks[jj][quarter * DQ + e], part);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        float x = part * a.scale_log2;
        if (has_bias) x += bias2 * (float)(j - qi);
        if (has_cap) x = cap2 * tanhf(x / cap2);   // cap tanh(s / cap), in log2 units
        const bool vis = mask_visible(a.mask, qi, j, doc_i, doc_row);
        if (!vis) continue;
        if (x > m_run) {
          const float alpha = fast_exp2(m_run - x);   // 0 when m_run = -inf
          l_run *= alpha;
#pragma unroll
          for (int e = 0; e < DQ; ++e) acc[e] *= alpha;
          m_run = x;
        }
        const float p = fast_exp2(x - m_run);
        l_run += p;
#pragma unroll
        for (int e = 0; e < DQ; ++e) acc[e] = fmaf(p, vs[jj][quarter * DQ + e], acc[e]);
      }
    }
  }

  if (row_ok) {
    const float inv = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int e = 0; e < DQ; ++e) a.out[q_base + (size_t)qi * D + quarter * DQ + e] = acc[e] * inv;
    if (quarter == 0) {
      a.lse[(size_t)(b * a.Hq + hq) * a.Sq + qi] =
          (l_run > 0.0f) ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    }
  }
}

template <int D>
hipError_t launch_d(const FwdParams &p, hipStream_t stream) {
  F32Args a;
  a.q = (const float *)p.q;
  a.k = (const float *)p.k;
  a.v = (const float *)p.v;
  a.out = (float *)p.out;
  a.lse = p.lse;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Skv = p.Skv;
  a.n_qtiles = (p.Sq + kRows - 1) / kRows;
  a.scale_log2 = p.scale * kLog2e;
  a.mask = p.mask;
  a.score = p.score;
  a.bm_num = p.bm_num;
  a.bm_idx = p.bm_idx;
  a.bm_nqb = p.bm_nqb;
  a.bm_nkb = p.bm_nkb;
  a.bm_batch = p.bm_batch;
  a.bm_kv_block = p.bm_kv_block;
  const unsigned grid = (unsigned)(a.n_qtiles * p.B * p.Hq);
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams &p, hipStream_t stream) {
  switch (p.D) {
    case 16: return launch_d<16>(p, stream);
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    case 256: return launch_d<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
