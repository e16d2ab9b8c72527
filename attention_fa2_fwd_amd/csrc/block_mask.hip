// BlockMask builder: for every (batch, query block, key block) decide whether
// any (i, j) in the block is visible (the block is listed) and whether all
// are (the block is flagged full), then write the ascending list per query
// block.  The FlexAttention write-up (introduction) names mask sparsity as
// what its kernel exploits; the list lets the forward kernel skip fully
// masked key tiles and drop the predicate on full ones.
//
// Visibility of a whole block follows from interval arithmetic for the
// position-only masks (over a block of rows [q0, q1] and columns [k0, k1]
// the difference i - j takes every integer value in [q0 - k1, q1 - k0]):
//   CAUSAL     any: k0 <= q1                  all: k1 <= q0
//   SLIDING    any: q1 - k0 >= 0 && q0 - k1 < W
//              all: q0 - k1 >= 0 && q1 - k0 < W
//   PREFIX_LM  any: k0 <= q1 || k0 < P        all: k1 < max(P, q0 + 1)
//   NONE       any and all
// DOCUMENT decides a block from the ids' summary where it can (blocks wholly
// above the diagonal, blocks that straddle it, id ranges that do not meet,
// blocks holding a single id) and otherwise scans for a shared id; no
// ordering of the ids is assumed.  DOCUMENT with a window (the AND of the two)
// takes the window's interval test first; where the window covers the whole
// block the document test decides, and where it covers part of it a scan of
// the pairs inside the window looks for a shared id.
//
// One workgroup per (batch, query block), one key block per thread; the list
// is compacted with wave ballots, 256 key blocks at a time.  Under DOCUMENT
// the workgroup first summarises every key block's ids (min, max) in LDS, so
// a key block's ids are read again only where the summary cannot decide.
#include "kernels.h"

namespace attn {
namespace {

constexpr int kThreads = 256;

struct BMArgs {
  MaskArgs mask;
  int Sq, Skv, q_block, kv_block, nqb, nkb;
  int32_t *num, *idx;
  uint8_t *full;
};

__device__ __forceinline__ void interval_block(const MaskArgs &m, int q0, int q1, int k0, int k1,
                                               bool &any, bool &all) {
  switch (m.kind) {
    case ATTN_MASK_NONE: any = true; all = true; break;
    case ATTN_MASK_CAUSAL: any = k0 <= q1; all = k1 <= q0; break;
    case ATTN_MASK_SLIDING:
      any = (q1 - k0 >= 0) && (q0 - k1 < m.window);
      all = (q0 - k1 >= 0) && (q1 - k0 < m.window);
      break;
    case ATTN_MASK_PREFIX_LM:
      any = (k0 <= q1) || (k0 < m.prefix_len);
      all = k1 < max(m.prefix_len, q0 + 1);
      break;
    default: any = false; all = false; break;
  }
}

// DOCUMENT flags of key block [k0, k1] against query block [q0, q1], whose
// ids are in qdoc with summary (qmin, qmax, q_uniform).  Blocks wholly above
// the diagonal hold no visible pair; blocks that straddle it hold (i, i);
// blocks wholly on or below it (k1 <= q0, every j <= i) are listed iff the
// two blocks share an id and full iff one id covers both.
// When ksum is set, it holds the key block's (min, max) id and whether the
// block holds any of the query block's ids, summarised beforehand, and the
// block is decided from it without reading the key ids again.
// qset holds the query block's ids with consecutive repeats dropped (nset of
// them): the same set of ids, for membership tests.
__device__ __forceinline__ void document_block(const int32_t *doc_row, const int32_t *qdoc,
                                               const int32_t *qset, int nset,
                                               int qmin, int qmax, bool q_uniform, int q0, int q1,
                                               int k0, int k1, bool &any, bool &all,
                                               const int4 *ksum = nullptr) {
  any = false;
  all = false;
  if (k0 > q1) return;
  if (k1 > q0) {
    any = true;
    return;
  }
  if (ksum) {
    // A shared id decides "any"; "all" needs one id on both sides.
    if (ksum->x > qmax || ksum->y < qmin || ksum->z == 0) return;
    any = true;
    all = q_uniform && ksum->x == ksum->y;
    return;
  }
  const int qval = qdoc[0];
  int kmin = doc_row[k0], kmax = kmin;
  bool k_uniform = true, hit_q = false;
  for (int j = k0; j <= k1; ++j) {
    const int d = doc_row[j];
    kmin = min(kmin, d);
    kmax = max(kmax, d);
    k_uniform &= (d == kmin) && (d == kmax);
    hit_q |= (d == qval);
  }
  if (kmax < qmin || kmin > qmax) return;
  if (q_uniform) {
    any = hit_q;
    all = k_uniform && hit_q;
    return;
  }
  if (k_uniform) {
    for (int t = 0; t < nset && !any; ++t) any = (qset[t] == kmin);
    return;
  }
  // General ids (not sorted, several per block): membership scan.
  for (int j = k0; j <= k1 && !any; ++j) {
    const int d = doc_row[j];
    if (d < qmin || d > qmax) continue;
    for (int t = 0; t < nset && !any; ++t) any = (qset[t] == d);
  }
}

// DOCUMENT and SLIDING together: a pair is visible when the ids agree and
// 0 <= i - j < W.
__device__ __forceinline__ void doc_window_block(const int32_t *doc_row, const int32_t *qdoc,
                                                 const int32_t *qset, int nset,
                                                 int qmin, int qmax, bool q_uniform, int window,
                                                 int q0, int q1, int k0, int k1, bool &any, bool &all,
                                                 const int4 *ksum = nullptr) {
  const bool w_any = (q1 - k0 >= 0) && (q0 - k1 < window);
  const bool w_all = (q0 - k1 >= 0) && (q1 - k0 < window);
  any = false;
  all = false;
  if (!w_any) return;
  bool d_any, d_all;
  document_block(doc_row, qdoc, qset, nset, qmin, qmax, q_uniform, q0, q1, k0, k1, d_any, d_all, ksum);
  if (!d_any) return;            // no pair with equal ids and j <= i at all
  if (w_all) {                   // every pair is inside the window
    any = true;
    all = d_all;
    return;
  }
  // The window covers part of the block: key j sees rows
  // max(q0, j) .. min(q1, j + W - 1); look there for its id, keys nearest
  // the diagonal first.
  for (int j = k1; j >= k0 && !any; --j) {
    const int d = doc_row[j];
    const int lo = max(q0, j);
    const int hi = min(q1, j + window - 1);
    for (int i = lo; i <= hi && !any; ++i) any = (qdoc[i - q0] == d);
  }
}

// Key blocks whose id summary is staged in LDS (more fall back to reading
// each key block's ids where they are needed).
constexpr int kSumCap = 1024;
// Distinct query ids up to which the summaries also record shared ids.
constexpr int kSetCap = 2;

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

__global__ __launch_bounds__(kThreads) void block_mask_kernel(BMArgs a) {
  __shared__ int32_t qdoc[1024];
  __shared__ int32_t qset[1024];          // qdoc with consecutive repeats dropped
  __shared__ int32_t nset_s;
  __shared__ int4 ksum[kSumCap];          // per key block: min id, max id, shares an id with qset
  __shared__ int32_t red[2][kThreads / 64];
  __shared__ int32_t wave_cnt[kThreads / 64];
  __shared__ int32_t running;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qb = blockIdx.x;
  const int b = blockIdx.y;
  const int q0 = qb * a.q_block;
  const int q1 = min(a.Sq, q0 + a.q_block) - 1;
  const int nq = q1 - q0 + 1;
  const bool doc = a.mask.kind == ATTN_MASK_DOCUMENT || a.mask.kind == kMaskDocWindow;
  const int32_t *doc_row = doc ? a.mask.doc_ids + (size_t)b * a.mask.doc_stride : nullptr;

  const size_t row = (size_t)b * a.nqb + qb;
  int32_t *idx_row = a.idx + row * a.nkb;
  uint8_t *full_row = a.full ? a.full + row * a.nkb : nullptr;

  // Query-block ids and their summary (min, max, all equal), then the
  // distinct ids in order of first appearance in runs (qset), then a summary
  // of every key block against them.
  int qmin = 0, qmax = 0;
  bool q_uniform = true;
  if (doc) {
    int lo = INT_MAX, hi = INT_MIN;
    for (int t = tid; t < nq; t += kThreads) {
      const int d = doc_row[q0 + t];
      qdoc[t] = d;
      lo = min(lo, d);
      hi = max(hi, d);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      red[0][wave] = lo;
      red[1][wave] = hi;
    }
    __syncthreads();
    qmin = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
    qmax = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    q_uniform = qmin == qmax;
    // The distinct runs of the query ids, compacted in order.
    if (tid == 0) nset_s = 0;
    __syncthreads();
    for (int base = 0; base < nq; base += kThreads) {
      const int t = base + tid;
      const bool start = t < nq && (t == 0 || qdoc[t] != qdoc[t - 1]);
      const unsigned long long ball = __ballot(start);
      const int rank_in_wave = __popcll(ball & ((1ull << lane) - 1ull));
      if (lane == 0) wave_cnt[wave] = __popcll(ball);
      __syncthreads();
      int off = nset_s;
      for (int w = 0; w < wave; ++w) off += wave_cnt[w];
      if (start) qset[off + rank_in_wave] = qdoc[t];
      __syncthreads();
      if (tid == 0) nset_s += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
      __syncthreads();
    }
  }
  const int nset = doc ? nset_s : 0;
  // The key blocks' summaries (only where the query block has few distinct
  // ids, as documents do; otherwise the blocks are decided from the ids).
  const bool use_sum = doc && a.nkb <= kSumCap && nset <= kSetCap;
  if (doc) {
    // The distinct ids in registers, padded with the first (a repeat tests
    // nothing new).
    int qs[kSetCap];
#pragma unroll
    for (int t = 0; t < kSetCap; ++t) {
      qs[t] = qset[t < nset ? t : 0];
      asm volatile("" : "+v"(qs[t]));   // held in VGPRs: as scalars they spill
    }
    // Counted in a VGPR: or-ing the compare masks instead keeps them in
    // scalar registers, which then spill.
    auto in_qset = [&](int d) __attribute__((always_inline)) -> int {
      int hit = 0;
#pragma unroll
      for (int t = 0; t < kSetCap; ++t) hit += (qs[t] == d) ? 1 : 0;
      return hit;
    };
    if (use_sum) {
      // Four threads per key block, each taking a quarter of its ids (a
      // multiple of 4, kv_block being a multiple of 16) in 16-byte loads
      // issued eight at a time, then a reduction over the four lanes.  Also
      // noted: whether the block holds any id of the query block.
      const bool vec = (reinterpret_cast<uintptr_t>(doc_row) & 15) == 0;
      const int part_len = a.kv_block / 4;
      for (int base = 0; base < a.nkb; base += kThreads / 4) {
        const int kb = base + tid / 4;
        const int part = tid % 4;
        int kl = INT_MAX, kh = INT_MIN;
        int hq = 0;
        if (kb < a.nkb) {
          const int k1 = min(a.Skv, (kb + 1) * a.kv_block) - 1;
          const int j0 = kb * a.kv_block + part * part_len;
          const int j1 = min(k1, j0 + part_len - 1);
          int j = j0;
          if (vec) {
            for (; j + 31 <= j1; j += 32) {
              int4 v[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) v[u] = *(const int4 *)(doc_row + j + 4 * u);
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                kl = min(kl, min(min(v[u].x, v[u].y), min(v[u].z, v[u].w)));
                kh = max(kh, max(max(v[u].x, v[u].y), max(v[u].z, v[u].w)));
                hq += in_qset(v[u].x) + in_qset(v[u].y) + in_qset(v[u].z) + in_qset(v[u].w);
              }
            }
            for (; j + 3 <= j1; j += 4) {
              const int4 v = *(const int4 *)(doc_row + j);
              kl = min(kl, min(min(v.x, v.y), min(v.z, v.w)));
              kh = max(kh, max(max(v.x, v.y), max(v.z, v.w)));
              hq += in_qset(v.x) + in_qset(v.y) + in_qset(v.z) + in_qset(v.w);
            }
          }
          for (; j <= j1; ++j) {
            const int d = doc_row[j];
            kl = min(kl, d);
            kh = max(kh, d);
            hq += in_qset(d);
          }
        }
        int hqi = hq > 0 ? 1 : 0;
        kl = min(kl, __shfl_xor(kl, 1));
        kh = max(kh, __shfl_xor(kh, 1));
        hqi |= __shfl_xor(hqi, 1);
        kl = min(kl, __shfl_xor(kl, 2));
        kh = max(kh, __shfl_xor(kh, 2));
        hqi |= __shfl_xor(hqi, 2);
        if (part == 0 && kb < a.nkb) ksum[kb] = make_int4(kl, kh, hqi, 0);
      }
    }
    __syncthreads();
  }
  if (tid == 0) running = 0;
  __syncthreads();

  for (int base = 0; base < a.nkb; base += kThreads) {
    // Flags of key blocks base .. base + 255, one block per thread.
    bool listed = false, full = false;
    const int kb = base + tid;
    if (kb < a.nkb) {
      const int k0 = kb * a.kv_block;
      const int k1 = min(a.Skv, k0 + a.kv_block) - 1;
      if (!doc)
        interval_block(a.mask, q0, q1, k0, k1, listed, full);
      else if (a.mask.kind == ATTN_MASK_DOCUMENT)
        document_block(doc_row, qdoc, qset, nset, qmin, qmax, q_uniform, q0, q1, k0, k1, listed, full,
                       use_sum ? &ksum[kb] : nullptr);
      else
        doc_window_block(doc_row, qdoc, qset, nset, qmin, qmax, q_uniform, a.mask.window, q0, q1, k0,
                         k1, listed, full, use_sum ? &ksum[kb] : nullptr);
    }

    // Compact: rank of this thread's listed block among listed blocks.
    const unsigned long long ball = __ballot(listed);
    const int rank_in_wave = __popcll(ball & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(ball);
    __syncthreads();
    int off = running;
    for (int w = 0; w < wave; ++w) off += wave_cnt[w];
    if (listed) {
      idx_row[off + rank_in_wave] = kb;
      if (full_row) full_row[off + rank_in_wave] = full ? 1 : 0;
    }
    __syncthreads();
    if (tid == 0) running += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    __syncthreads();
  }

  const int count = running;
  for (int n = count + tid; n < a.nkb; n += kThreads) {
    idx_row[n] = -1;
    if (full_row) full_row[n] = 0;
  }
  if (tid == 0) a.num[row] = count;
}

// The lists by key block: one workgroup per (batch, key block), one query
// block per thread.  A query block lists key block kb if its ascending row
// list holds kb (binary search); the column is compacted with the same wave
// ballots, so it comes out ascending.
struct BMTArgs {
  const int32_t *num, *idx;
  const uint8_t *full;
  int32_t *q_num, *q_idx;
  uint8_t *q_full;
  int nqb, nkb;
};

__global__ __launch_bounds__(kThreads) void block_mask_transpose_kernel(BMTArgs a) {
  __shared__ int32_t wave_cnt[kThreads / 64];
  __shared__ int32_t running;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kb = blockIdx.x;
  const int b = blockIdx.y;
  const size_t col = (size_t)b * a.nkb + kb;
  int32_t *idx_col = a.q_idx + col * a.nqb;
  uint8_t *full_col = a.q_full ? a.q_full + col * a.nqb : nullptr;
  if (tid == 0) running = 0;
  __syncthreads();
  for (int base = 0; base < a.nqb; base += kThreads) {
    const int qb = base + tid;
    bool listed = false, full = false;
    if (qb < a.nqb) {
      const size_t row = (size_t)b * a.nqb + qb;
      const int n = min(max(a.num[row], 0), a.nkb);
      const int32_t *list = a.idx + row * a.nkb;
      int lo = 0, hi = n - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const int v = list[mid];
        if (v == kb) {
          listed = true;
          full = a.full && a.full[row * a.nkb + mid] != 0;
          break;
        }
        if (v < kb) lo = mid + 1; else hi = mid - 1;
      }
    }
    const unsigned long long ball = __ballot(listed);
    const int rank_in_wave = __popcll(ball & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(ball);
    __syncthreads();
    int off = running;
    for (int w = 0; w < wave; ++w) off += wave_cnt[w];
    if (listed) {
      idx_col[off + rank_in_wave] = qb;
      if (full_col) full_col[off + rank_in_wave] = full ? 1 : 0;
    }
    __syncthreads();
    if (tid == 0) running += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    __syncthreads();
  }
  const int count = running;
  for (int n = count + tid; n < a.nqb; n += kThreads) {
    idx_col[n] = -1;
    if (full_col) full_col[n] = 0;
  }
  if (tid == 0) a.q_num[col] = count;
}

}  // namespace

hipError_t launch_block_mask_transpose(const BlockMaskTransposeParams &p, hipStream_t stream) {
  BMTArgs a;
  a.num = p.num;
  a.idx = p.idx;
  a.full = p.full;
  a.q_num = p.q_num;
  a.q_idx = p.q_idx;
  a.q_full = p.q_full;
  a.nqb = p.nqb;
  a.nkb = p.nkb;
  hipLaunchKernelGGL(block_mask_transpose_kernel, dim3(p.nkb, p.batch), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_block_mask(const BlockMaskParams &p, hipStream_t stream) {
  BMArgs a;
  a.mask = p.mask;
  a.Sq = p.Sq;
  a.Skv = p.Skv;
  a.q_block = p.q_block;
  a.kv_block = p.kv_block;
  a.nqb = p.nqb;
  a.nkb = p.nkb;
  a.num = p.num;
  a.idx = p.idx;
  a.full = p.full;
  hipLaunchKernelGGL(block_mask_kernel, dim3(p.nqb, p.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
