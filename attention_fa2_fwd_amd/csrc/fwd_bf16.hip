// Fused attention forward, bf16 inputs, MFMA on gfx950 (CDNA4).
//
// One pass over the visible key tiles with an online softmax (running row
// max and row sum, rescaled when the max grows; LSE written at the end) —
// the 1-pass FlashAttention form of "Attention优化｜2w字原理&图解: 从
// Online-Softmax到FlashAttention V1/V2/V3" (abstract), in FA2-style tiling:
// a workgroup owns a tile of query rows and streams K/V tiles through LDS.
// Score modifiers and mask predicates are applied inside the tile loop, as
// the FlexAttention write-up describes for its fused kernel (§相对位置编码:
// the bias is computed in-kernel, no S x S tensor), and fully masked key
// tiles are never visited (its introduction: mask sparsity is exploited).
//
// Layout of the work (CDNA4-specific choices):
//  * workgroup = 256 threads = 4 wave64s, 128 query rows; each wave owns 32
//    consecutive rows.  Key tiles of 64 rows.  Two workgroups per CU.
//  * Scores are computed transposed, S^T = K·Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand, Q^T (kept in
//    VGPRs for the whole kernel) the B operand.  In the 32x32 accumulator
//    layout a lane then holds one query column and 16 keys, so the row max
//    and row sum of the softmax are in-lane reductions plus one exchange
//    between the two 32-lane halves, not 32-lane shuffles.
//  * P^T leaves the accumulator already in the B-operand layout of the next
//    MFMA, O^T += V^T·P^T, with the key order inside each 16-key chunk
//    permuted identically on both operands; V^T fragments are read from the
//    row-major V tile with ds_read_b64_tr_b16 (the gfx950 transposing LDS
//    read), so V is never transposed in memory.
//  * exp2 with scale·log2(e) folded into one multiply; LSE converted to the
//    natural log on output.
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are
//    issued before the current tile's MFMAs.  Rows are padded (K by 16 B, V
//    by 64 B) so the 16-byte and transposed LDS reads do not collide in banks.
//  * Causal-type masks: workgroups with the most key tiles are launched
//    first; waves skip tiles that hold no visible key for their rows and
//    skip the predicate on tiles where every key is visible.
#include "kernels.h"

namespace attn {
namespace {

constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // key rows per tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kListCap = 512;  // BlockMask entries staged in LDS per query tile
// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct FwdCfg {
  static constexpr int KS = D + 8;    // K row stride in LDS (elements)
  static constexpr int VS = D + 32;   // V row stride in LDS (elements)
  static constexpr int KTILE = kBN * KS;
  static constexpr int VTILE = kBN * VS;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int NDC = D / 16;            // 16-wide d chunks of S^T = K Q^T
  static constexpr int NDB = D / 32;            // 32-row d blocks of O^T
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int LOADS = kBN * CPR / kThreads;
  static_assert(kBN * CPR % kThreads == 0, "tile load mapping");
};

struct KernelArgs {
  const __bf16 *q, *k, *v;
  void *out;           // bf16 or fp32 [B, Hq, Sq, D]
  float *lse;
  int B, Hq, Hkv, Sq, Skv;
  int n_qtiles;
  float scale_log2;    // scale * log2(e)
  MaskArgs mask;
  ScoreArgs score;
  const int32_t *bm_num, *bm_idx;
  const uint8_t *bm_full;
  int bm_nqb, bm_nkb, bm_batch, tiles_per_block;
};

__device__ __forceinline__ s16x4 lds_read_tr(const __bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
}

// Compile-time variants: D, the mask kind, GEN (materialise the modified
// score x = c*s + bias before the max: needed for a bias or a scale <= 0) and
// the output dtype.  Without GEN the row max is taken on the raw dot products
// (c > 0 preserves order) and p = 2^(c*s - m) is one FMA and one exp2.
template <int D, int MASK, bool GEN, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(KernelArgs a) {
  using C = FwdCfg<D>;
  extern __shared__ __align__(16) __bf16 smem[];
  __shared__ __align__(16) int32_t kdoc[2][kBN];   // document ids of the staged key tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;      // lane half: selects keys 4h..4h+3 of each 8
  const int l32 = lane & 31;    // query column of this lane

  // Heaviest query tiles first (causal-type masks give later tiles more keys).
  const int bh_count = a.B * a.Hq;
  const int qt = a.n_qtiles - 1 - (int)(blockIdx.x / bh_count);
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hkv = (hq * a.Hkv) / a.Hq;
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * 32;
  const int qw1 = min(qw0 + 31, a.Sq - 1);
  const int qi = qw0 + l32;

  const size_t q_base = ((size_t)(b * a.Hq + hq) * a.Sq) * D;
  const size_t kv_base = ((size_t)(b * a.Hkv + hkv) * a.Skv) * D;
  const __bf16 *Kg = a.k + kv_base;
  const __bf16 *Vg = a.v + kv_base;

  // Q^T fragments: lane holds Q[qi][16c + 8h .. 16c + 8h + 7] (rows past Sq
  // read row Sq-1 and are never stored).  The empty asm statements make the
  // loads complete here, so the tile loop never waits on them.
  bf16x8 qf[C::NDC];
  {
    const bf16x8 *src = (const bf16x8 *)(a.q + q_base + (size_t)min(qi, a.Sq - 1) * D);
#pragma unroll
    for (int c = 0; c < C::NDC; ++c) qf[c] = src[2 * c + h];
#pragma unroll
    for (int c = 0; c < C::NDC; ++c) asm volatile("" ::"v"(qf[c]));
  }

  // ---- key tiles to visit.  A BlockMask row is staged in LDS (its first
  // kListCap entries) so the tile loop reads it without touching the vector
  // memory counters.
  __shared__ int32_t s_blk[kListCap];
  __shared__ uint8_t s_full[kListCap];
  const int qlast = min(q0 + kBM, a.Sq) - 1;
  int n_tiles;
  int t_first = 0;
  const int32_t *bm_list = nullptr;
  const uint8_t *bm_flags = nullptr;
  if (a.bm_num) {
    const int bb = (a.bm_batch == 1) ? 0 : b;
    const size_t row = (size_t)bb * a.bm_nqb + qt;
    // Counts and indices are device data: clamp them so a malformed list
    // can only drop tiles, never address outside K/V.
    const int n_blocks = min(max(a.bm_num[row], 0), a.bm_nkb);
    n_tiles = n_blocks * a.tiles_per_block;
    bm_list = a.bm_idx + row * a.bm_nkb;
    if (a.bm_full) bm_flags = a.bm_full + row * a.bm_nkb;
    for (int t = tid; t < min(n_blocks, kListCap); t += kThreads) {
      s_blk[t] = bm_list[t];
      s_full[t] = bm_flags ? bm_flags[t] : 0;
    }
    __syncthreads();   // the list is read by every wave from here on
  } else {
    int lo = 0, hi = a.Skv;
    if (MASK == ATTN_MASK_CAUSAL || MASK == ATTN_MASK_DOCUMENT) {
      hi = min(a.Skv, qlast + 1);
    } else if (MASK == ATTN_MASK_SLIDING) {
      hi = min(a.Skv, qlast + 1);
      lo = max(0, q0 - a.mask.window + 1);
    } else if (MASK == ATTN_MASK_PREFIX_LM) {
      hi = min(a.Skv, max(qlast + 1, a.mask.prefix_len));
    }
    t_first = lo / kBN;
    n_tiles = (hi > lo) ? (hi + kBN - 1) / kBN - t_first : 0;
  }
  auto tile_key0 = [&](int n) -> int {
    if (bm_list) {
      const int bi = n / a.tiles_per_block;
      const int blk = (bi < kListCap) ? s_blk[bi] : bm_list[bi];
      if (blk < 0 || blk >= a.bm_nkb) return a.Skv;      // treated as an empty tile
      return blk * (a.tiles_per_block * kBN) + (n % a.tiles_per_block) * kBN;
    }
    return (t_first + n) * kBN;
  };
  auto tile_block_full = [&](int n) -> bool {
    if (!bm_flags) return false;
    const int bi = n / a.tiles_per_block;
    return ((bi < kListCap) ? s_full[bi] : bm_flags[bi]) != 0;
  };

  const int32_t *doc_row = (MASK == ATTN_MASK_DOCUMENT) ? a.mask.doc_ids + (size_t)b * a.mask.doc_stride
                                                        : nullptr;

  // ---- global -> register -> LDS staging of one K/V tile through raw
  // buffer loads: rows past Skv fall outside the buffer's range and read as
  // zero, so the ragged last tile needs no branch.
  const __amdgpu_buffer_rsrc_t k_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)Kg, (short)0, a.Skv * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)Vg, (short)0, a.Skv * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t d_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(doc_row ? doc_row : a.mask.doc_ids), (short)0, doc_row ? a.Skv * 4 : 0, kBufferFlags);
  u32x4 kreg[C::LOADS], vreg[C::LOADS];
  int32_t dreg = 0;
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = i * kThreads + tid;
      const int off = ((k0 + c / C::CPR) * D + (c % C::CPR) * 8) * 2;
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, off, 0, 0);
      vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, off, 0, 0);
    }
    if (MASK == ATTN_MASK_DOCUMENT && tid < kBN)
      dreg = __builtin_amdgcn_raw_buffer_load_b32(d_rsrc, (k0 + tid) * 4, 0, 0);
  };
  auto lstore = [&](int buf) {
    __bf16 *Ks = smem + buf * C::STAGE;
    __bf16 *Vs = Ks + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / C::CPR;
      const int col = (c % C::CPR) * 8;
      *(u32x4 *)(Ks + row * C::KS + col) = kreg[i];
      *(u32x4 *)(Vs + row * C::VS + col) = vreg[i];
    }
    if (MASK == ATTN_MASK_DOCUMENT && tid < kBN) kdoc[buf][tid] = dreg;
  };

  // Per-row softmax state.  m_run: the reference max of the log2-domain
  // scores (identical in both lane halves), raised only when a tile's max
  // exceeds it by more than kTau, so p = 2^(x - m_run) <= 2^kTau; l_run: this
  // half's share of the row sum.
  constexpr float kTau = 8.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x16 o[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) o[i] = f32x16{};

  const float c_log2 = a.scale_log2;
  const float bias2 = GEN ? bias_coeff(a.score, hq, a.Hq) * kLog2e : 0.0f;
  const int doc_i = (MASK == ATTN_MASK_DOCUMENT) ? doc_row[min(qi, a.Sq - 1)] : 0;
  asm volatile("" ::"v"(doc_i));   // complete the load before the tile loop

  // V^T fragment addressing for ds_read_b64_tr_b16: within each 16-lane
  // group, lanes 4r..4r+3 point at 4 consecutive d of key row r; the read
  // hands lane i the 4 keys' values at d = i.
  const int tr_g = lane >> 4;
  const int tr_j = lane & 15;
  const int tr_key = 4 * h + (tr_j >> 2);                 // + 16c (+8 for the second read)
  const int tr_d = 16 * (tr_g & 1) + 4 * (tr_j & 3);      // + 32 dblk

  if (n_tiles > 0) {
    gload(tile_key0(0));
    lstore(0);
  }
  __syncthreads();

  for (int n = 0; n < n_tiles; ++n) {
    const int cur = n & 1;
    const int k0 = tile_key0(n);
    if (n + 1 < n_tiles) gload(tile_key0(n + 1));

    // Does this wave have any visible key in the tile, and are all visible?
    bool empty = (qw0 >= a.Sq) || (k0 >= a.Skv);
    bool full = (k0 + kBN <= a.Skv);
    if (MASK == ATTN_MASK_CAUSAL || MASK == ATTN_MASK_DOCUMENT) {
      empty = empty || (k0 > qw1);
      full = full && (k0 + kBN - 1 <= qw0);
      if (MASK == ATTN_MASK_DOCUMENT) full = full && tile_block_full(n);
    } else if (MASK == ATTN_MASK_SLIDING) {
      empty = empty || (k0 > qw1) || (qw0 - (k0 + kBN - 1) >= a.mask.window);
      full = full && (k0 + kBN - 1 <= qw0) && (qw1 - k0 < a.mask.window);
    } else if (MASK == ATTN_MASK_PREFIX_LM) {
      empty = empty || ((k0 > qw1) && (k0 >= a.mask.prefix_len));
      full = full && ((k0 + kBN - 1 <= qw0) || (k0 + kBN <= a.mask.prefix_len));
    }

    if (!empty) {
      const __bf16 *Ks = smem + cur * C::STAGE;
      const __bf16 *Vs = Ks + C::KTILE;

      // S^T = K Q^T for two 32-key blocks.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const __bf16 *krow = Ks + (kb * 32 + l32) * C::KS + 8 * h;
#pragma unroll
        for (int c = 0; c < C::NDC; ++c) {
          const bf16x8 ka = *(const bf16x8 *)(krow + 16 * c);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s[kb], 0, 0, 0);
        }
      }

      // Accumulator element r of block kb is key j = jb + kb*32 + 8(r/4) + r%4
      // with jb = k0 + 4h.
      const int jb = k0 + 4 * h;
      if constexpr (GEN) {
        const float cb = bias2 * (float)(jb - qi);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float off = (float)(kb * 32 + 8 * (r >> 2) + (r & 3));
            s[kb][r] = __builtin_fmaf(s[kb][r], c_log2, __builtin_fmaf(bias2, off, cb));
          }
      }
      if (!full) {
        // Partial tile: the mask predicate per element; -inf where hidden
        // (for the raw scores too: c > 0 on that path).
        const int dq = qi - jb;                       // j <= qi  <=>  off <= dq
        int32_t kd[2][4][4];
        if (MASK == ATTN_MASK_DOCUMENT) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int4 t = *(const int4 *)&kdoc[cur][kb * 32 + 8 * g + 4 * h];
              kd[kb][g][0] = t.x; kd[kb][g][1] = t.y; kd[kb][g][2] = t.z; kd[kb][g][3] = t.w;
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
            bool vis = off < a.Skv - jb;
            if (MASK == ATTN_MASK_CAUSAL) vis = vis && (off <= dq);
            if (MASK == ATTN_MASK_SLIDING) vis = vis && (off <= dq) && (dq - off < a.mask.window);
            if (MASK == ATTN_MASK_PREFIX_LM) vis = vis && ((off <= dq) || (off < a.mask.prefix_len - jb));
            if (MASK == ATTN_MASK_DOCUMENT) vis = vis && (off <= dq) && (kd[kb][r >> 2][r & 3] == doc_i);
            s[kb][r] = vis ? s[kb][r] : -INFINITY;
          }
      }

      // Tile row max (raw or modified scores), shared by the two halves.
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) tmax = fmaxf(tmax, fmaxf(s[kb][r], s[kb][r + 1]));
      if constexpr (!GEN) tmax *= c_log2;
      tmax = half_swap_max(tmax);

      // Raise the reference max only past the threshold (wave-uniform branch).
      const bool need = tmax > m_run + kTau;
      if (__any(need)) {
        const float m_new = need ? tmax : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;   // 0 when m_run = -inf
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < C::NDB; ++i) o[i] *= alpha;
      }
      const float mu = (m_run == -INFINITY) ? 0.0f : m_run;

      // P = 2^(x - m), packed to bf16 pairs in the B-operand order.
      uint32_t pk[2][8];
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0, p1;
          if constexpr (GEN) {
            p0 = fast_exp2(s[kb][r] - mu);
            p1 = fast_exp2(s[kb][r + 1] - mu);
          } else {
            p0 = fast_exp2(__builtin_fmaf(s[kb][r], c_log2, -mu));
            p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c_log2, -mu));
          }
          psum += p0 + p1;
          pk[kb][r >> 1] = pack_bf16x2(p0, p1);
        }
      l_run += psum;

      // O^T += V^T P^T over four 16-key chunks.
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 pw = {pk[c >> 1][4 * (c & 1) + 0], pk[c >> 1][4 * (c & 1) + 1],
                          pk[c >> 1][4 * (c & 1) + 2], pk[c >> 1][4 * (c & 1) + 3]};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const __bf16 *vbase = Vs + (16 * c + tr_key) * C::VS + tr_d;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const s16x4 lo = lds_read_tr(vbase + 32 * db);
          const s16x4 hi = lds_read_tr(vbase + 8 * C::VS + 32 * db);
          const u32x4 vw = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                            __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pb,
                                                          o[db], 0, 0, 0);
        }
      }
    }

    if (n + 1 < n_tiles) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l, LSE = (m + log2 l) ln 2.
  const float l_tot = half_swap_sum(l_run);
  if (qi < a.Sq) {
    const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
    if constexpr (OUT_F32) {
      float *orow = (float *)a.out + q_base + (size_t)qi * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 w = {o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv,
                           o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
          *(f32x4 *)(orow + 32 * db + 8 * g + 4 * h) = w;
        }
      }
    } else {
      __bf16 *orow = (__bf16 *)a.out + q_base + (size_t)qi * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w = {pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                           pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
          *(u32x2 *)(orow + 32 * db + 8 * g + 4 * h) = w;
        }
      }
    }
    if (h == 0) {
      a.lse[(size_t)(b * a.Hq + hq) * a.Sq + qi] =
          (l_tot > 0.0f) ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int MASK, bool GEN, bool OUT_F32>
hipError_t launch_variant(const KernelArgs &a, unsigned grid, hipStream_t stream) {
  using C = FwdCfg<D>;
  static bool attr_set = false;  // the attribute is per function; set once
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)fwd_bf16_kernel<D, MASK, GEN, OUT_F32>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, MASK, GEN, OUT_F32>), dim3(grid), dim3(kThreads),
                     C::LDS_BYTES, stream, a);
  return hipGetLastError();
}

template <int D, bool GEN, bool OUT_F32>
hipError_t launch_mask(const KernelArgs &a, int mask, unsigned grid, hipStream_t stream) {
  switch (mask) {
    case ATTN_MASK_NONE: return launch_variant<D, ATTN_MASK_NONE, GEN, OUT_F32>(a, grid, stream);
    case ATTN_MASK_CAUSAL: return launch_variant<D, ATTN_MASK_CAUSAL, GEN, OUT_F32>(a, grid, stream);
    case ATTN_MASK_SLIDING: return launch_variant<D, ATTN_MASK_SLIDING, GEN, OUT_F32>(a, grid, stream);
    case ATTN_MASK_PREFIX_LM: return launch_variant<D, ATTN_MASK_PREFIX_LM, GEN, OUT_F32>(a, grid, stream);
    case ATTN_MASK_DOCUMENT: return launch_variant<D, ATTN_MASK_DOCUMENT, GEN, OUT_F32>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_d(const FwdParams &p, hipStream_t stream) {
  KernelArgs a;
  a.q = (const __bf16 *)p.q;
  a.k = (const __bf16 *)p.k;
  a.v = (const __bf16 *)p.v;
  a.out = p.out;
  a.lse = p.lse;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Skv = p.Skv;
  a.n_qtiles = (p.Sq + kBM - 1) / kBM;
  a.scale_log2 = p.scale * kLog2e;
  a.mask = p.mask;
  a.score = p.score;
  a.bm_num = p.bm_num;
  a.bm_idx = p.bm_idx;
  a.bm_full = p.bm_full;
  a.bm_nqb = p.bm_nqb;
  a.bm_nkb = p.bm_nkb;
  a.bm_batch = p.bm_batch;
  a.tiles_per_block = p.bm_num ? p.bm_kv_block / kBN : 1;
  const unsigned grid = (unsigned)(a.n_qtiles * p.B * p.Hq);
  // The raw-score path needs a positive scale and no bias.
  const bool gen = (p.score.kind != ATTN_SCORE_NONE) || !(a.scale_log2 > 0.0f);
  if (gen) {
    return p.out_f32 ? launch_mask<D, true, true>(a, p.mask.kind, grid, stream)
                     : launch_mask<D, true, false>(a, p.mask.kind, grid, stream);
  }
  return p.out_f32 ? launch_mask<D, false, true>(a, p.mask.kind, grid, stream)
                   : launch_mask<D, false, false>(a, p.mask.kind, grid, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams &p, hipStream_t stream) {
  if (p.D == 64) return launch_d<64>(p, stream);
  if (p.D == 128) return launch_d<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
