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
// DOCUMENT compares document ids element by element (no ordering of the ids
// is assumed), after rejecting blocks that lie wholly above the diagonal.
//
// One workgroup per (batch, query block); the list is compacted with wave
// ballots, 256 key blocks at a time.
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

__global__ __launch_bounds__(kThreads) void block_mask_kernel(BMArgs a) {
  __shared__ int32_t qdoc[1024];
  __shared__ int32_t kdoc[1024];
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
  const bool doc = a.mask.kind == ATTN_MASK_DOCUMENT;
  const int32_t *doc_row = doc ? a.mask.doc_ids + (size_t)b * a.mask.doc_stride : nullptr;

  const size_t row = (size_t)b * a.nqb + qb;
  int32_t *idx_row = a.idx + row * a.nkb;
  uint8_t *full_row = a.full ? a.full + row * a.nkb : nullptr;

  if (doc) {
    for (int t = tid; t < nq; t += kThreads) qdoc[t] = doc_row[q0 + t];
  }
  if (tid == 0) running = 0;
  __syncthreads();

  for (int base = 0; base < a.nkb; base += kThreads) {
    // Flags of key blocks base .. base + 255: one block per thread for the
    // interval kinds; DOCUMENT scans each block with the whole workgroup.
    bool listed = false, full = false;
    const int kb = base + tid;
    if (!doc) {
      if (kb < a.nkb) {
        const int k0 = kb * a.kv_block;
        const int k1 = min(a.Skv, k0 + a.kv_block) - 1;
        interval_block(a.mask, q0, q1, k0, k1, listed, full);
      }
    } else {
      const int kend = min(a.nkb, base + kThreads);
      for (int kk = base; kk < kend; ++kk) {
        const int k0 = kk * a.kv_block;
        const int k1 = min(a.Skv, k0 + a.kv_block) - 1;
        const int nk = k1 - k0 + 1;
        bool any_vis = false, all_vis = false;
        if (k0 <= q1) {
          __syncthreads();
          for (int t = tid; t < nk; t += kThreads) kdoc[t] = doc_row[k0 + t];
          __syncthreads();
          int any_l = 0, all_l = 1;
          const int pairs = nq * nk;
          for (int pidx = tid; pidx < pairs; pidx += kThreads) {
            const int ii = pidx / nk;
            const int jj = pidx - ii * nk;
            const bool v = (k0 + jj <= q0 + ii) && (kdoc[jj] == qdoc[ii]);
            any_l |= v;
            all_l &= v;
          }
          any_vis = __syncthreads_or(any_l) != 0;
          all_vis = __syncthreads_and(all_l) != 0;
        }
        if (kk == kb) {
          listed = any_vis;
          full = all_vis;
        }
      }
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

}  // namespace

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
