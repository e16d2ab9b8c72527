// Attention backward from the stored LSE, bf16 inputs, fp32 gradients, MFMA
// on gfx950 (CDNA4).
//
// The FlexAttention write-up ("新PyTorch API：几行代码实现不同注意力变体，兼具
// FlashAttention性能和PyTorch灵活性") produces its backward by automatic
// differentiation of the forward (introduction) and describes it as
// deterministic, recomputing more intermediates than FlashAttention-2
// (§性能).  This backward follows that description: no atomics, every
// gradient element written by one workgroup, and P recomputed from the
// forward's LSE wherever it is needed.  With x = s Q K^T, S = score_mod(x)
// masked, P = softmax(S) = exp(S - LSE):
//
//   D_i = sum_d dO_id O_id                       (bwd_dq_kernel, stored)
//   dP  = dO V^T,  dS = P (dP - D),  dX = dS score_mod'(x)
//   dQ  = s dX K                                 (bwd_dq_kernel)
//   dV  = P^T dO,  dK = s dX^T Q                 (bwd_dkdv_kernel, after it)
//
// The two main kernels reuse the forward kernel's MFMA conventions
// (v_mfma_f32_32x32x16_bf16, 4 waves x 32 rows, LDS tiles of 1 KiB blocks
// filled by buffer_load ... lds), but read each streamed tile both row-wise
// and through the transposing ds_read_b64_tr_b16, so their tiles place rows
// and permute chunks to keep both kinds of read free of bank conflicts
// (Tile below):
//  * bwd_dq_kernel, one workgroup per (b, hq, 128 query rows) (with groups
//    of four or more query heads and no BlockMask, per 32 positions of four
//    heads sharing a kv head, one head per wave), streams 64-key tiles of K
//    and V.  S^T = K Q^T and dP^T = V dO^T take K and V rows from
//    LDS as the A operand and Q^T, dO^T from registers as the B operand; the
//    lane then holds one query and 16 keys, so LSE and D are one register
//    each, and dS^T leaves the accumulator already in the B-operand layout of
//    dQ^T += K^T dS^T, whose A operand is the transposed read of the K tile.
//    It also forms each row's D from its O and dO rows and stores it.
//  * bwd_dkdv_kernel, one workgroup per (b, hkv, 128 keys), streams 32-row
//    tiles of Q and dO for every query head of the GQA group, so dK and dV
//    sum the group in registers.  S = Q K^T and dP = dO V^T take Q and dO
//    rows from LDS, K from registers and V from a per-wave LDS copy; the lane
//    then holds one key, P and dS are already the B operands of
//    dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read transposed
//    from the same LDS tiles.  Per-query LSE and D are staged in LDS with the
//    tile.
// Tiles without a visible pair are skipped and the predicate is dropped on
// tiles where every pair is visible, from the mask's closed-form bounds or,
// given a BlockMask, from its lists: by query block for the dQ pass, by key
// block for the dK/dV pass, staged in LDS.  Under document masks the dQ pass
// also compares each key tile's document-id range with its wave's.  The tiles with the most work
// launch first in both passes (with a BlockMask, ranked by list length).
#include "kernels.h"

// Every fused multiply-add here is written as one: with implicit
// contraction the compiler fused a product into a later sum in some
// places and not in others, depending on how the surrounding code was
// laid out, so equal formulas could round differently between builds.
#pragma clang fp contract(off)

namespace attn {
namespace {

constexpr int kThreads = 256;
// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;
constexpr int kQRows = 128;        // query rows per dQ workgroup
constexpr int kKTile = 64;         // key rows per tile in the dQ kernel
constexpr int kKRows = 128;        // keys per dK/dV workgroup
constexpr int kQTile = 32;         // query rows per tile in the dK/dV kernel
constexpr int kListCap = 1024;     // BlockMask entries staged in LDS (host-checked)
// Score forms: raw scores, a bias added, or the soft cap.
constexpr int kModAdd = 0, kModCap = 1, kModRaw = 2;

typedef __attribute__((address_space(3))) void lds_void;

// LDS tile of ROWS rows of D bf16.  The LDS DMA fills it in 1 KiB blocks
// (load i of wave w fills block 4i + w, its lane L bytes 16L .. 16L + 15),
// and it is read two ways: 16-byte row reads, whose 16-lane passes read 16
// consecutive rows at one chunk, and transposing reads, whose 32-lane passes
// read 64 bytes of each of 4 consecutive rows.  LDS has 64 banks of 4 bytes,
// so a row-read pass is free of conflicts when its 16 rows put the chunk on
// 16 distinct 16-byte bank slots, and a transposing pass when its 4 rows
// start on slots 4 apart.  Rows are placed in blocks and slots, and the
// 16-byte chunks of row q permuted as chunk ^ xr(q), so that both hold:
//  - D = 128 (4 rows per block): row q = 16c + 8a + 4h + j sits in block
//    2j + a (+ 8h in a 16-block tile) at slot c (2c + h in an 8-block
//    tile), chunks XOR h; blocks 1056 bytes apart put block b on slot 2b.
//  - D = 64 (8 rows per block): row q sits in block q % NB at slot q / NB,
//    chunks XOR (q / 4) % 4; blocks 1088 bytes apart put block b on slot 4b.
// In both, each lane's read addresses are one base per kind of read plus
// compile-time steps, and the loads of a wave are one offset plus
// compile-time changes; check() verifies this for every lane.
template <int D, int ROWS>
struct Tile {
  static constexpr int ROWB = D * 2;
  static constexpr int NB = ROWS * ROWB / 1024;     // blocks
  static constexpr int SPB = 1024 / ROWB;           // rows per block
  static constexpr bool PERM = D == 128;
  static constexpr int BLK = PERM ? 1024 + 32 : 1024 + 64;
  static constexpr int BYTES = NB * BLK;
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int LOADS = NB / 4;              // direct loads per wave per tile
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(NB % 4 == 0 && 32 % NB == 0 && (NB <= 8 || NB == 16), "row block mapping");
  static_assert(!PERM || NB == 8 || NB == 16, "D = 128 placement");

  static constexpr int blk(int q) {
    return PERM ? 2 * (q & 3) + ((q >> 3) & 1) + (NB == 16 ? 8 * ((q >> 2) & 1) : 0) : q % NB;
  }
  static constexpr int slot(int q) { return PERM ? (NB == 16 ? q >> 4 : 2 * (q >> 4) + ((q >> 2) & 1)) : q / NB; }
  static constexpr int xr(int q) { return PERM ? (q >> 2) & 1 : (q >> 2) & 3; }
  static constexpr int row_off(int q) { return blk(q) * BLK + slot(q) * ROWB; }
  static constexpr int row_at(int b, int s) {
    if (!PERM) return b + NB * s;
    const int h = NB == 16 ? b >> 3 : s & 1, c = NB == 16 ? s : s >> 1;
    return 16 * c + 8 * (b & 1) + 4 * h + ((b >> 1) & 3);
  }
  // Source byte offset (from the tile's first row) of lane L's 16 bytes in
  // load i of wave w; load i's equals (load 0's ^ 16 lxor(i)) + i RSTEP.
  static constexpr int src(int w, int L, int i) {
    const int q = row_at(4 * i + w, L / CPR);
    return q * ROWB + 16 * ((L % CPR) ^ xr(q));
  }
  static constexpr int RSTEP = PERM ? 2 * ROWB : 4 * ROWB;
  static constexpr int lxor(int i) { return PERM ? (NB == 16 ? i >> 1 : 0) : i; }
  // Row reads: lane (h, l32) reads row l32 + 32 kb, chunk 2c + h at
  // row_base(l32, h, c % 2) + row_step(kb) + 32c.
  static constexpr int row_base_def(int l32, int h, int e) {
    return row_off(l32) + 16 * ((2 * e + h) ^ xr(l32)) - 32 * e;
  }
  static constexpr int row_step(int kb) { return row_off(32 * kb) - row_off(0); }
  // Transposing reads: within each 16-lane group, lanes 4r .. 4r + 3 point at
  // 4 consecutive d of row 16c + 8 hi + 4h + r (d = 32 ((lane >> 4) & 1) +
  // 4 (lane & 3) + 32 db), at tr_base(lane, hi) + tr_step(c, hi) + 64 db.
  static constexpr int tr_base_def(int lane, int hi) {
    const int tj = lane & 15, r = 8 * hi + 4 * (lane >> 5) + (tj >> 2);
    return row_off(r) + 16 * ((2 * ((lane >> 4) & 1) + ((tj & 3) >> 1)) ^ xr(r)) + 8 * (tj & 1);
  }
  static constexpr int tr_step(int c, int hi) { return row_off(16 * c + 8 * hi) - row_off(8 * hi); }
  // The D = 128 placement needs one base of each kind (the XOR flips only
  // the chunk bit a lane's h gives; row 8 + r sits one block after row r);
  // written so, the compiler keeps one register for each.
  static constexpr int row_base(int l32, int h, int e) { return row_base_def(l32, h, PERM ? 0 : e); }
  static constexpr int tr_base(int lane, int hi) { return PERM ? tr_base_def(lane, 0) + hi * BLK : tr_base_def(lane, hi); }

  static constexpr bool check() {
    bool seen[ROWS] = {};
    for (int q = 0; q < ROWS; ++q) {
      if (blk(q) >= NB || slot(q) >= SPB || row_at(blk(q), slot(q)) != q || seen[q]) return false;
      seen[q] = true;
    }
    for (int w = 0; w < 4; ++w)
      for (int L = 0; L < 64; ++L)
        for (int i = 0; i < LOADS; ++i)
          if (src(w, L, i) != ((src(w, L, 0) ^ (16 * lxor(i))) + i * RSTEP)) return false;
    for (int kb = 0; kb < ROWS / 32; ++kb)
      for (int l = 0; l < 32; ++l)
        if (row_off(32 * kb + l) - row_off(l) != row_step(kb) || xr(32 * kb + l) != xr(l)) return false;
    for (int c = 0; c < ROWS / 16; ++c)
      for (int r = 0; r < 16; ++r)
        if (row_off(16 * c + r) - row_off(r) != tr_step(c, r >> 3) || xr(16 * c + r) != xr(r)) return false;
    for (int lane = 0; lane < 64; ++lane)
      for (int e = 0; e < 2; ++e)
        if (row_base(lane & 31, lane >> 5, e) != row_base_def(lane & 31, lane >> 5, e) ||
            tr_base(lane, e) != tr_base_def(lane, e))
          return false;
    return true;
  }
};
static_assert(Tile<64, 32>::check() && Tile<64, 64>::check() && Tile<128, 32>::check() &&
                  Tile<128, 64>::check(),
              "LDS tile placement");

struct BwdArgs {
  const __bf16 *q, *k, *v, *out, *dout;
  const float *lse;
  float *row_dot;   // D per query row: written by the dQ kernel, read by the dK/dV kernel
  float *dq, *dk, *dv;
  int B, Hq, Hkv, Sq, Skv;
  float scale, scale_log2;
  MaskArgs mask;
  ScoreArgs score;
  // BlockMask (bm_num == nullptr: closed-form tile ranges), 128 x 128 blocks
  const int32_t *bm_num, *bm_idx, *bm_qnum, *bm_qidx;
  const uint8_t *bm_full, *bm_qfull;
  int bm_nqb, bm_nkb, bm_batch;
  int gqa_pack;   // 1: a dQ workgroup is 32 positions of four query heads sharing a kv head
};

__device__ __forceinline__ s16x4 lds_read_tr(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}

// visible(i, j) of the mask kind, given the two document ids when the kind
// compares them.
template <int MASK>
__device__ __forceinline__ bool pair_visible(const MaskArgs &m, int i, int j, int doc_i, int doc_j) {
  if (MASK == ATTN_MASK_NONE) return true;
  if (MASK == ATTN_MASK_CAUSAL) return j <= i;
  if (MASK == ATTN_MASK_SLIDING) return (j <= i) && (i - j < m.window);
  if (MASK == ATTN_MASK_PREFIX_LM) return (j <= i) || (j < m.prefix_len);
  if (MASK == ATTN_MASK_DOCUMENT) return (j <= i) && (doc_i == doc_j);
  if (MASK == kMaskDocWindow) return (j <= i) && (i - j < m.window) && (doc_i == doc_j);
  return false;
}

// Visibility class of the block of queries [i0, i1] x keys [j0, j1]:
// no visible pair (empty) or every pair visible (full), from the mask's
// bounds.  Document masks are never full here (no id summaries).
template <int MASK>
__device__ __forceinline__ bool block_empty(const MaskArgs &m, int i0, int i1, int j0, int j1) {
  if (MASK == ATTN_MASK_CAUSAL || MASK == ATTN_MASK_DOCUMENT) return j0 > i1;
  if (MASK == ATTN_MASK_SLIDING || MASK == kMaskDocWindow) return (j0 > i1) || (i0 - j1 >= m.window);
  if (MASK == ATTN_MASK_PREFIX_LM) return (j0 > i1) && (j0 >= m.prefix_len);
  return false;
}
template <int MASK>
__device__ __forceinline__ bool block_full(const MaskArgs &m, int i0, int i1, int j0, int j1) {
  if (MASK == ATTN_MASK_NONE) return true;
  if (MASK == ATTN_MASK_CAUSAL) return j1 <= i0;
  if (MASK == ATTN_MASK_SLIDING) return (j1 <= i0) && (i1 - j0 < m.window);
  if (MASK == ATTN_MASK_PREFIX_LM) return (j1 <= i0) || (j1 < m.prefix_len);
  return false;
}

// Bias coefficient of query head hq (wave-uniform) with a slope table read
// through the scalar cache: a wait for it then never waits for the vector
// loads in flight.
__device__ __forceinline__ float bias_coeff_uniform(const ScoreArgs &s, int hq, int Hq) {
  if (s.kind == ATTN_SCORE_ALIBI && s.slopes) {
    typedef __attribute__((address_space(4))) const float *const_f32p;
    return ((const_f32p)s.slopes)[__builtin_amdgcn_readfirstlane(hq)];
  }
  return bias_coeff(s, hq, Hq);
}

// Log2-domain modified score of raw dot product s, and the factor
// score_mod'(x) of the chain rule.  With a bias, bias2 (j - i) is passed as
// base + bias2 * off: base per tile and lane, off a compile-time offset of
// the accumulator element, so the bias costs one FMA.  (Where only log2 P is
// needed, the kernels fold the LSE into base instead.)
template <int MOD>
__device__ __forceinline__ float mod_score(float s, float c_log2, float bias2, float cap_k, float cap2,
                                           float base, float off) {
  if (MOD == kModCap) return softcap_log2_fast(s, cap_k, cap2);
  if (MOD == kModRaw) return s * c_log2;
  return __builtin_fmaf(s, c_log2, __builtin_fmaf(bias2, off, base));
}
// log2 P = x - LSE (log2 units); for raw scores x = c s, taken as one FMA.
template <int MOD>
__device__ __forceinline__ float log2_p_arg(float s, float c_log2, float x, float lse2) {
  return (MOD == kModRaw) ? __builtin_fmaf(s, c_log2, -lse2) : x - lse2;
}
template <int MOD>
__device__ __forceinline__ float mod_grad(float x, float inv_cap2) {
  if (MOD == kModCap) {
    const float t = x * inv_cap2;   // tanh of the scaled score
    return __builtin_fmaf(-t, t, 1.0f);
  }
  return 1.0f;
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, hq, 128 query rows); wave w owns rows
// q0 + 32w .. + 31, lane (h, l32) the query q0 + 32w + l32.
template <int D, int MASK, int MOD>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  using T = Tile<D, kKTile>;
  constexpr int NDC = D / 16, NDB = D / 32;
  constexpr bool DOC = MASK == ATTN_MASK_DOCUMENT || MASK == kMaskDocWindow;
  constexpr bool WIN = MASK == ATTN_MASK_SLIDING || MASK == kMaskDocWindow;
  __shared__ __align__(16) char k_lds0[T::BYTES];
  __shared__ __align__(16) char k_lds1[T::BYTES];
  __shared__ __align__(16) char v_lds0[T::BYTES];
  __shared__ __align__(16) char v_lds1[T::BYTES];
  // Document ids of a staged key tile, then their min and max.
  __shared__ __align__(16) int32_t kdoc0[kKTile + 4];
  __shared__ __align__(16) int32_t kdoc1[kKTile + 4];
  __shared__ __align__(16) int32_t s_blk[kListCap];
  __shared__ uint8_t s_full[kListCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Rows of the workgroup: 128 consecutive rows of one head, wave w taking
  // rows 32w .. 32w + 31; or, with gqa_pack (Hq / Hkv a multiple of 4, no
  // BlockMask), 32 positions of four heads sharing a kv head, wave w taking
  // head 4g + w, so every wave needs the same key tiles.
  const int pack = a.gqa_pack;
  const int rows = pack ? 32 : kQRows;
  const int n_qtiles = (a.Sq + rows - 1) / rows;
  const int hunits = pack ? a.Hq / 4 : a.Hq;
  const int bh_count = a.B * hunits;
  // Workgroups go round-robin to the 8 XCDs; each XCD gets a contiguous run
  // of head units, so the query heads of one kv head share an L2.
  const int xh = (int)(blockIdx.x % bh_count);
  const int bh = (bh_count % 8 == 0) ? (xh % 8) * (bh_count / 8) + xh / 8 : xh;
  const int b = bh / hunits;
  const int hu = bh - b * hunits;
  const int hq = pack ? 4 * hu + __builtin_amdgcn_readfirstlane(tid >> 6) : hu;
  // Longest key ranges first: the later query tiles, or with a BlockMask the
  // tiles with the most listed blocks (each wave ranks the counts itself).
  const int pos = (int)(blockIdx.x / bh_count);
  int qt = n_qtiles - 1 - pos;
  int n_ranked = -1;   // the tile's clamped list length, when the ranking ran
  if (a.bm_num && n_qtiles <= kOrderCap) {
    const int bb = (a.bm_batch == 1) ? 0 : b;
    qt = work_ordered_tile(a.bm_num + (size_t)bb * a.bm_nqb, n_qtiles, min(a.bm_nkb, kListCap), pos, true,
                           &n_ranked);
  }
  const int hkv = (hq * a.Hkv) / a.Hq;
  const int q0 = qt * rows;
  const int qw0 = pack ? q0 : q0 + wave * 32;
  const int qw1 = min(qw0 + 31, a.Sq - 1);
  const int qi = qw0 + l32;
  const int qr = min(qi, a.Sq - 1);

  const size_t q_base = ((size_t)(b * a.Hq + hq) * a.Sq) * D;
  const size_t kv_base = ((size_t)(b * a.Hkv + hkv) * a.Skv) * D;

  // Q^T and dO^T fragments (B operands): lane holds X[qi][16c + 8h .. + 7];
  // O the same way, for the row term below.
  bf16x8 qf[NDC], df[NDC], of[NDC];
  {
    const bf16x8 *qs = (const bf16x8 *)(a.q + q_base + (size_t)qr * D);
    const bf16x8 *ds = (const bf16x8 *)(a.dout + q_base + (size_t)qr * D);
    const bf16x8 *os = (const bf16x8 *)(a.out + q_base + (size_t)qr * D);
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      qf[c] = qs[2 * c + h];
      df[c] = ds[2 * c + h];
      of[c] = os[2 * c + h];
    }
  }
  const size_t row = (size_t)(b * a.Hq + hq) * a.Sq + qr;
  const float lse_row = a.lse[row];
  const int32_t *doc_row = DOC ? a.mask.doc_ids + (size_t)b * a.mask.doc_stride : nullptr;
  const int doc_i = DOC ? doc_row[qr] : 0;

  // Key tiles of the workgroup's rows: the BlockMask row of this 128-row
  // query block (two 64-key tiles per listed block), or a closed-form range.
  // The row loads above are in flight while the list is staged: the two
  // share one memory latency.
  const bool use_bm = a.bm_num != nullptr;
  int n_tiles = 0, t_first = 0;
  if (use_bm) {
    const int bb = (a.bm_batch == 1) ? 0 : b;
    const size_t brow = (size_t)bb * a.bm_nqb + qt;
    // Counts and indices are device data: clamped, so a malformed list can
    // only drop tiles, never address outside K / V.
    int n_blocks = __builtin_amdgcn_readfirstlane(n_ranked);
    if (n_blocks < 0) n_blocks = min(max(a.bm_num[brow], 0), min(a.bm_nkb, kListCap));
    n_tiles = 2 * n_blocks;
    stage_list_row<kListCap, kThreads>(a.bm_idx + brow * a.bm_nkb,
                                       a.bm_full ? a.bm_full + brow * a.bm_nkb : nullptr, n_blocks, s_blk,
                                       s_full, tid);
    __syncthreads();
  } else {
    const int qlast = min(q0 + rows, a.Sq) - 1;
    int lo = 0, hi = a.Skv;
    if (MASK == ATTN_MASK_CAUSAL || MASK == ATTN_MASK_DOCUMENT) {
      hi = min(a.Skv, qlast + 1);
    } else if (WIN) {
      hi = min(a.Skv, qlast + 1);
      lo = max(0, q0 - a.mask.window + 1);
    } else if (MASK == ATTN_MASK_PREFIX_LM) {
      hi = min(a.Skv, max(qlast + 1, a.mask.prefix_len));
    }
    t_first = lo / kKTile;
    n_tiles = (hi > lo) ? (hi + kKTile - 1) / kKTile - t_first : 0;
  }
  const float lse2 = lse_row * kLog2e;
  // D = sum_d dO O over the row: each lane half holds every other 8-wide
  // chunk of it.  Stored for the dK/dV kernel.
  float dsum;
  {
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)of[c][e], (float)df[c][e], part);
    }
    dsum = part + __shfl_xor(part, 32);
  }
  // Range of the wave's document ids (rows past Sq repeat row Sq - 1).
  const int dmin_w = DOC ? wave_min_i32(doc_i) : 0;
  const int dmax_w = DOC ? wave_max_i32(doc_i) : 0;
  // Wave 0 stages a key tile's ids (one per lane) with their min and max.
  auto store_kdoc = [&](int32_t *dst, int id) __attribute__((always_inline)) {
    dst[lane] = id;
    const int mn = wave_min_i32(id), mx = wave_max_i32(id);
    if (lane == 0) {
      dst[kKTile] = mn;
      dst[kKTile + 1] = mx;
    }
  };
  if (h == 0 && qi < a.Sq) a.row_dot[row] = dsum;
  const float c_log2 = a.scale_log2;
  const float bias2 = (MOD == kModAdd) ? bias_coeff(a.score, hq, a.Hq) * kLog2e : 0.0f;
  const float cap2 = (MOD == kModCap) ? a.score.softcap * kLog2e : 0.0f;
  const float cap_k = (MOD == kModCap) ? (2.0f / a.score.softcap) * c_log2 : 0.0f;
  const float inv_cap2 = (MOD == kModCap) ? 1.0f / cap2 : 0.0f;

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

  auto tile_key0 = [&](int n) __attribute__((always_inline)) -> int {
    if (use_bm) {
      const int blk = s_blk[n >> 1];
      if (blk < 0 || blk >= a.bm_nkb) return a.Skv;   // an empty tile
      return blk * 128 + (n & 1) * kKTile;
    }
    return (t_first + n) * kKTile;
  };
  auto tile_flag = [&](int n) __attribute__((always_inline)) -> bool { return use_bm && s_full[n >> 1] != 0; };

  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.k + kv_base), (short)0, a.Skv * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.v + kv_base), (short)0, a.Skv * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t d_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(doc_row ? doc_row : a.mask.doc_ids), (short)0, doc_row ? a.Skv * 4 : 0, kBufferFlags);
  const int ld_off = T::src(wave, lane, 0);
  auto load_tile = [&](char *dst, __amdgpu_buffer_rsrc_t rs, int row0) __attribute__((always_inline)) {
    const int soff = __builtin_amdgcn_readfirstlane(row0 * D * 2);
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      // (A type-dependent expression among this builtin's arguments makes
      // the host pass drop the kernel's launch stub: offsets are computed
      // first.)
      const int vo = (ld_off ^ (16 * T::lxor(i))) + i * T::RSTEP;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (4 * i + wave) * T::BLK), 16, vo, soff, 0, 0);
    }
  };
  auto load_doc = [&](int key0) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_raw_buffer_load_b32(d_rsrc, lane * 4, __builtin_amdgcn_readfirstlane(key0 * 4), 0);
  };

  // Row reads (A operand, keys 32 kb + l32, d chunk 2c + h) and transposed
  // reads (A operand K^T: the first and second 8 keys of each 16-key chunk).
  const int rd_row0 = T::row_base(l32, h, 0), rd_row1 = T::row_base(l32, h, 1);
  const int rd_tr0 = T::tr_base(lane, 0), rd_tr1 = T::tr_base(lane, 1);

  auto tile_step = [&](int k0, bool flag, const char *kt, const char *vt, const int32_t *kdoc)
      __attribute__((always_inline)) {
    if (block_empty<MASK>(a.mask, qw0, qw1, k0, k0 + kKTile - 1) || qw0 >= a.Sq || k0 >= a.Skv) return;
    // Document masks: a tile whose id range misses the wave's holds no
    // visible pair; one whose ids and the wave's are all one id is visible
    // wherever the position part allows (no id test per element).
    bool one_id = false;
    if (DOC) {
      const int kmn = kdoc[kKTile], kmx = kdoc[kKTile + 1];
      if (kmx < dmin_w || kmn > dmax_w) return;
      one_id = (kmn == kmx) && (dmin_w == dmax_w) && (kmn == dmin_w);
    }
    const bool pos_full = (MASK == ATTN_MASK_DOCUMENT) ? (k0 + kKTile - 1 <= qw0)
                        : (MASK == kMaskDocWindow) ? ((k0 + kKTile - 1 <= qw0) && (qw1 - k0 < a.mask.window))
                        : false;
    // Wave-uniform by construction; readfirstlane tells the compiler so, and
    // the test below becomes one branch per tile instead of an exec-mask
    // branch around every score.
    const bool full = __builtin_amdgcn_readfirstlane(
        (flag || block_full<MASK>(a.mask, qw0, qw1, k0, k0 + kKTile - 1) || (one_id && pos_full)) &&
        (k0 + kKTile <= a.Skv));
    // S^T and dP^T for the two 32-key blocks.
    f32x16 s[2], dp[2];
    // The K and V fragments of chunk n = NDC kb + c are read LAQ chunks ahead
    // of their products (the D = 128 soft-cap variants have no registers for
    // it).
    constexpr int LAQ = (D == 128 && MOD == kModCap) ? 0 : 1, NQ = 2 * NDC;
    struct QOps {
      bf16x8 k, v;
    };
    auto rd_q = [&](int n) __attribute__((always_inline)) -> QOps {
      const int kb = n / NDC, c = n % NDC;
      const int o = ((c & 1) ? rd_row1 : rd_row0) + T::row_step(kb) + 32 * c;
      return QOps{*(const bf16x8 *)(kt + o), *(const bf16x8 *)(vt + o)};
    };
    QOps qq[LAQ + 1];
#pragma unroll
    for (int n = 0; n < LAQ; ++n) qq[n] = rd_q(n);
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int kb = n / NDC, c = n % NDC;
      if (c == 0) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
      }
      if (n + LAQ < NQ) qq[(n + LAQ) % (LAQ + 1)] = rd_q(n + LAQ);
      if (LAQ > 0) __builtin_amdgcn_sched_barrier(0);
      const QOps &x = qq[n % (LAQ + 1)];
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x.k, qf[c], s[kb], 0, 0, 0);
      dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x.v, df[c], dp[kb], 0, 0, 0);
      if (LAQ > 0) __builtin_amdgcn_sched_barrier(0);
    }
    // dS^T element r of block kb: key j = k0 + 32 kb + 8 (r / 4) + 4h + r % 4.
    const int jb = k0 + 4 * h;
    const float bias_base = bias2 * (float)(jb - qi);   // j - i = (jb - qi) + off
    // With a bias, log2 P = c s + bias2 off + (bias_base - LSE): the row's
    // LSE goes into the tile's base, two FMAs per score.
    const float base_lse = bias_base - lse2;
    int4 kd4 = int4{0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
        const int j = jb + off;
        const float x = mod_score<MOD>(s[kb][r], c_log2, bias2, cap_k, cap2, bias_base, (float)off);
        float p = fast_exp2((MOD == kModAdd) ? mod_score<MOD>(s[kb][r], c_log2, bias2, cap_k, cap2, base_lse, (float)off)
                                             : log2_p_arg<MOD>(s[kb][r], c_log2, x, lse2));
        if (!full) {
          // The keys' document ids, four at a time (keys off .. off + 3 of
          // the group are consecutive): one LDS read per four scores.
          if (DOC && (r & 3) == 0) kd4 = *(const int4 *)(kdoc + 4 * h + off);
          const int doc_j = !DOC ? 0 : (r & 3) == 0 ? kd4.x : (r & 3) == 1 ? kd4.y : (r & 3) == 2 ? kd4.z : kd4.w;
          const bool vis = (j < a.Skv) && pair_visible<MASK>(a.mask, qi, j, doc_i, doc_j);
          p = vis ? p : 0.0f;
        }
        s[kb][r] = p * (dp[kb][r] - dsum) * mod_grad<MOD>(x, inv_cap2);
      }
    // dQ^T += K^T dS^T, 16 keys at a time, at D = 64 at raised wave
    // priority: the wave feeding the matrix cores issues ahead of the other
    // wave's elementwise work (measured 6-9% faster on the causal D=64
    // backward; at D = 128 the GQA window backward ran 2.6-2.8% faster
    // without it).
    if (D == 64) __builtin_amdgcn_s_setprio(1);
    const char *kbase0 = kt + rd_tr0, *kbase1 = kt + rd_tr1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      asm volatile("" ::: "memory");   // keep this chunk's LDS reads in the chunk
      const int kb = c >> 1;
      const int r0 = 8 * (c & 1);
      const u32x4 pw = {pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]), pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]),
                        pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]), pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7])};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const s16x4 lo4 = lds_read_tr(kbase0 + T::tr_step(c, 0) + 64 * db);
        const s16x4 hi4 = lds_read_tr(kbase1 + T::tr_step(c, 1) + 64 * db);
        const u32x4 kw = {__builtin_bit_cast(u32x2, lo4)[0], __builtin_bit_cast(u32x2, lo4)[1],
                          __builtin_bit_cast(u32x2, hi4)[0], __builtin_bit_cast(u32x2, hi4)[1]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kw), pb, acc[db], 0, 0, 0);
      }
    }
    if (D == 64) __builtin_amdgcn_s_setprio(0);
  };

  // Double-buffered tile loop: iteration n loads tile n + 1 into the buffers
  // tile n - 1 used, computes tile n, then waits for its loads and meets
  // the other waves at the barrier.
  if (n_tiles > 0) {
    load_tile(k_lds0, k_rsrc, tile_key0(0));
    load_tile(v_lds0, v_rsrc, tile_key0(0));
    if (DOC && wave == 0) store_kdoc(kdoc0, load_doc(tile_key0(0)));
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  // The current tile's first key and full flag are carried from the
  // iteration that loaded it, so an iteration looks up one list entry.
  int key_cur = (n_tiles > 0) ? __builtin_amdgcn_readfirstlane(tile_key0(0)) : 0;
  bool flag_cur = (n_tiles > 0) && tile_flag(0);
  auto iteration = [&](int n, char *k_cur, char *v_cur, int32_t *d_cur, char *k_nxt, char *v_nxt,
                       int32_t *d_nxt) __attribute__((always_inline)) {
    const int k0 = key_cur;
    const bool f0 = flag_cur;
    int doc_fill = 0;
    if (n + 1 < n_tiles) {
      const int k1 = __builtin_amdgcn_readfirstlane(tile_key0(n + 1));
      key_cur = k1;
      flag_cur = tile_flag(n + 1);
      load_tile(k_nxt, k_rsrc, k1);
      load_tile(v_nxt, v_rsrc, k1);
      if (DOC && wave == 0) doc_fill = load_doc(k1);
    }
    if (n < n_tiles) tile_step(k0, f0, k_cur, v_cur, d_cur);
    if (DOC && wave == 0 && n + 1 < n_tiles) store_kdoc(d_nxt, doc_fill);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Tiles in pairs; an odd count ends with an empty visit (its barrier
  // only), so the tile body is built twice rather than three times.
  for (int n = 0; n < n_tiles; n += 2) {
    iteration(n, k_lds0, v_lds0, kdoc0, k_lds1, v_lds1, kdoc1);
    iteration(n + 1, k_lds1, v_lds1, kdoc1, k_lds0, v_lds0, kdoc0);
  }

  // dQ = s dX K: lane holds dQ^T[32 db + 8 g + 4h + e][qi].
  if (qi < a.Sq) {
    float *orow = a.dq + q_base + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 w = {acc[db][4 * g + 0] * a.scale, acc[db][4 * g + 1] * a.scale,
                         acc[db][4 * g + 2] * a.scale, acc[db][4 * g + 3] * a.scale};
        *(f32x4 *)(orow + 32 * db + 8 * g + 4 * h) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (b, hkv, 128 keys); wave w owns keys
// j0 + 32w .. + 31, lane (h, l32) the key j0 + 32w + l32.
template <int D, int MASK, int MOD>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(BwdArgs a) {
  using T = Tile<D, kQTile>;
  constexpr int NDC = D / 16, NDB = D / 32;
  constexpr bool DOC = MASK == ATTN_MASK_DOCUMENT || MASK == kMaskDocWindow;
  constexpr bool WIN = MASK == ATTN_MASK_SLIDING || MASK == kMaskDocWindow;
  __shared__ __align__(16) char q_lds0[T::BYTES];
  __shared__ __align__(16) char q_lds1[T::BYTES];
  __shared__ __align__(16) char o_lds0[T::BYTES];   // dO tiles
  __shared__ __align__(16) char o_lds1[T::BYTES];
  // Per-query values of the staged tile: LSE (log2 units), D, document id.
  __shared__ __align__(16) float qv_lse0[kQTile], qv_lse1[kQTile];
  __shared__ __align__(16) float qv_dot0[kQTile], qv_dot1[kQTile];
  __shared__ __align__(16) int32_t qv_doc0[kQTile], qv_doc1[kQTile];
  // V rows of each wave's 32 keys (the B operand of dP = dO V^T), read from
  // LDS rather than held in registers; rows padded by 16 bytes so the 16
  // lanes of a read group hit distinct banks.
  constexpr int VROW = D * 2 + 16;
  __shared__ __align__(16) char v_rows[4][32 * VROW];
  __shared__ __align__(16) int32_t s_qblk[kListCap];
  __shared__ uint8_t s_qfull[kListCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int bh_count = a.B * a.Hkv;
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / a.Hkv;
  const int hkv = bh - b * a.Hkv;
  // Most query tiles first: the first key tiles, or with a BlockMask the key
  // blocks with the most listed query blocks (ties, the earlier block first;
  // each wave ranks the counts itself).
  const int pos = (int)(blockIdx.x / bh_count);
  int kt = pos;
  int n_ranked = -1;   // the block's clamped list length, when the ranking ran
  if (a.bm_num && a.bm_qnum) {
    const int n_ktiles = (a.Skv + kKRows - 1) / kKRows;
    if (n_ktiles <= kOrderCap) {
      const int bb = (a.bm_batch == 1) ? 0 : b;
      kt = work_ordered_tile(a.bm_qnum + (size_t)bb * a.bm_nkb, n_ktiles, min(a.bm_nqb, kListCap), pos,
                             false, &n_ranked);
    }
  }
  const int G = a.Hq / a.Hkv;
  const int j0 = kt * kKRows;
  const int jw0 = j0 + wave * 32;
  const int jw1 = jw0 + 31;
  const int kj = jw0 + l32;
  const int kr = min(kj, a.Skv - 1);
  const int jlast = min(j0 + kKRows, a.Skv) - 1;

  const size_t kv_base = ((size_t)(b * a.Hkv + hkv) * a.Skv) * D;
  // K rows as B operands in registers: lane holds K[kj][16c + 8h .. + 7].
  // V rows go to this wave's LDS rows (32 rows x D, 16-byte chunks, rows
  // past Skv repeat the last one); they are first read after the barrier
  // that follows the prologue's loads.
  bf16x8 kf[NDC];
  constexpr int CPR = D / 8;
  constexpr int VPL = 32 * CPR / 64;   // 16-byte V chunks per lane
  bf16x8 vx[VPL];
  {
    const bf16x8 *ks = (const bf16x8 *)(a.k + kv_base + (size_t)kr * D);
#pragma unroll
    for (int c = 0; c < NDC; ++c) kf[c] = ks[2 * c + h];
#pragma unroll
    for (int t = 0; t < VPL; ++t) {
      const int idx = 64 * t + lane;
      const int r = idx / CPR, ch = idx % CPR;
      const int key = min(jw0 + r, a.Skv - 1);
      vx[t] = *(const bf16x8 *)(a.v + kv_base + (size_t)key * D + 8 * ch);
    }
  }
  const int32_t *doc_row = DOC ? a.mask.doc_ids + (size_t)b * a.mask.doc_stride : nullptr;
  const int doc_j = DOC ? doc_row[kr] : 0;

  // Query tiles that may see the workgroup's keys [j0, jlast]: the
  // BlockMask column of this 128-key block (four 32-row tiles per listed
  // query block), or a closed-form range.  The K and V row loads above are
  // in flight while the list is staged: the two share one memory latency.
  const bool use_bm = a.bm_num != nullptr;
  int n_qt = 0, t_first = 0;
  if (use_bm) {
    const int bb = (a.bm_batch == 1) ? 0 : b;
    const size_t bcol = (size_t)bb * a.bm_nkb + kt;
    int n_blocks = __builtin_amdgcn_readfirstlane(n_ranked);
    if (n_blocks < 0) n_blocks = min(max(a.bm_qnum[bcol], 0), min(a.bm_nqb, kListCap));
    n_qt = 4 * n_blocks;
    stage_list_row<kListCap, kThreads>(a.bm_qidx + bcol * a.bm_nqb,
                                       a.bm_qfull ? a.bm_qfull + bcol * a.bm_nqb : nullptr, n_blocks, s_qblk,
                                       s_qfull, tid);
    __syncthreads();
  } else {
    int lo = 0, hi = a.Sq - 1;
    if (MASK == ATTN_MASK_CAUSAL || MASK == ATTN_MASK_DOCUMENT) {
      lo = j0;
    } else if (WIN) {
      lo = j0;
      hi = min(a.Sq - 1, jlast + a.mask.window - 1);
    } else if (MASK == ATTN_MASK_PREFIX_LM) {
      lo = (j0 < a.mask.prefix_len) ? 0 : j0;
    }
    t_first = lo / kQTile;
    n_qt = (hi >= lo) ? hi / kQTile + 1 - t_first : 0;
  }
#pragma unroll
  for (int t = 0; t < VPL; ++t) {
    const int idx = 64 * t + lane;
    *(bf16x8 *)(v_rows[wave] + (idx / CPR) * VROW + 16 * (idx % CPR)) = vx[t];
  }
  const char *vrow = v_rows[wave] + l32 * VROW + 16 * h;
  const float c_log2 = a.scale_log2;
  const float cap2 = (MOD == kModCap) ? a.score.softcap * kLog2e : 0.0f;
  const float cap_k = (MOD == kModCap) ? (2.0f / a.score.softcap) * c_log2 : 0.0f;
  const float inv_cap2 = (MOD == kModCap) ? 1.0f / cap2 : 0.0f;

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const int n_iter = n_qt * G;   // (query head, query tile) pairs

  // Loads of a (head, tile) pair: Q and dO rows into LDS by buffer_load ...
  // lds (rows past Sq read as zero), the per-query values by wave 0.
  const int ld_off = T::src(wave, lane, 0);
  // A step is one (query head, query tile) pair, heads outer; steps advance
  // one at a time, so finding a step's head and tile needs no division.
  struct Step {
    int hq, t;
  };
  auto next_step = [&](Step st) __attribute__((always_inline)) -> Step {
    return (st.t + 1 < n_qt) ? Step{st.hq, st.t + 1} : Step{st.hq + 1, 0};
  };
  auto tile_q0 = [&](int t) __attribute__((always_inline)) -> int {
    if (use_bm) {
      const int blk = s_qblk[t >> 2];
      if (blk < 0 || blk >= a.bm_nqb) return a.Sq;   // rows past Sq: no effect
      return blk * 128 + (t & 3) * kQTile;
    }
    return (t_first + t) * kQTile;
  };
  auto tile_flag = [&](int t) __attribute__((always_inline)) -> bool {
    return use_bm && s_qfull[t >> 2] != 0;
  };
  auto load_tiles = [&](Step st, int q0, char *qd, char *od) __attribute__((always_inline)) {
    const int hq = st.hq;
    const size_t base = ((size_t)(b * a.Hq + hq) * a.Sq) * D;
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.q + base), (short)0, a.Sq * D * 2, kBufferFlags);
    const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.dout + base), (short)0, a.Sq * D * 2, kBufferFlags);
    const int soff = __builtin_amdgcn_readfirstlane(q0 * D * 2);
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int vo = (ld_off ^ (16 * T::lxor(i))) + i * T::RSTEP;   // (see the dQ kernel's loads)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void *)(qd + (4 * i + wave) * T::BLK), 16, vo, soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(orr, (lds_void *)(od + (4 * i + wave) * T::BLK), 16, vo, soff, 0, 0);
    }
  };
  // Per-query values for lane < 32 of wave 0: LSE (+inf past Sq, so p = 0
  // there), D, document id.  The LSE goes to log2 units only when it is
  // stored, after the step's work: converting it where it is fetched makes
  // the wave wait there for its load, and with it for the next tiles' loads.
  // (An empty asm keeps the compiler from moving the product back up.)
  struct QVals {
    float lse, dot;
    int doc;
  };
  auto fetch_qvals = [&](Step st, int q0) __attribute__((always_inline)) -> QVals {
    const int i = q0 + lane;
    QVals r{INFINITY, 0.0f, -1};
    if (lane < kQTile && i < a.Sq) {
      const size_t row = (size_t)(b * a.Hq + st.hq) * a.Sq + i;
      r.lse = a.lse[row];
      r.dot = a.row_dot[row];
      if (DOC) r.doc = doc_row[i];
    }
    return r;
  };
  // With a bias the staged value also carries the query part of the bias,
  // bias2 (i - j0) for query i = q0s + lane (bias2 the step's coefficient in
  // log2 units); j0 keeps both parts small where pairs are near.
  auto store_qvals = [&](const QVals &r, float *ls, float *dt, int32_t *dc, int q0s, float bias2s)
      __attribute__((always_inline)) {
    if (lane < kQTile) {
      float lse = r.lse;
      asm volatile("" : "+v"(lse));
      const float lse2 = lse * kLog2e;
      ls[lane] = (MOD == kModAdd) ? __builtin_fmaf(bias2s, (float)(q0s + lane - j0), lse2) : lse2;
      dt[lane] = r.dot;
      if (DOC) dc[lane] = r.doc;
    }
  };

  const int rd_row0 = T::row_base(l32, h, 0), rd_row1 = T::row_base(l32, h, 1);
  const int rd_tr0 = T::tr_base(lane, 0), rd_tr1 = T::tr_base(lane, 1);

  auto tile_step = [&](int i0, bool flag, float bias2, const char *qt_, const char *ot, const float *ls,
                       const float *dt,
                       const int32_t *dc) __attribute__((always_inline)) {
    const int i1 = i0 + kQTile - 1;
    if (jw0 >= a.Skv || i0 >= a.Sq || block_empty<MASK>(a.mask, i0, i1, jw0, jw1)) return;
    const bool full = flag || block_full<MASK>(a.mask, i0, i1, jw0, jw1);
    // S = Q K^T and dP = dO V^T for the 32 queries: element r is query
    // i0 + 8 (r / 4) + 4h + r % 4, key kj.
    f32x16 s = f32x16{}, dp = f32x16{};
    // Each chunk's Q, dO and V fragments are read LAS chunks ahead of their
    // products, so the LDS latency is not waited out product by product (the
    // D = 128 document variants with a bias have no registers for it).
    constexpr int LAS = (D == 128 && DOC && MOD == kModAdd) ? 0 : 1;
    struct SOps {
      bf16x8 q, o, v;
    };
    auto rd_s = [&](int c) __attribute__((always_inline)) -> SOps {
      const int o = ((c & 1) ? rd_row1 : rd_row0) + 32 * c;
      return SOps{*(const bf16x8 *)(qt_ + o), *(const bf16x8 *)(ot + o), *(const bf16x8 *)(vrow + 32 * c)};
    };
    SOps sq[LAS + 1];
#pragma unroll
    for (int c = 0; c < LAS; ++c) sq[c] = rd_s(c);
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      if (c + LAS < NDC) sq[(c + LAS) % (LAS + 1)] = rd_s(c + LAS);
      if (LAS > 0) __builtin_amdgcn_sched_barrier(0);
      const SOps &x = sq[c % (LAS + 1)];
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x.q, kf[c], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x.o, x.v, dp, 0, 0, 0);
      if (LAS > 0) __builtin_amdgcn_sched_barrier(0);
    }
    // P and dS go to bf16 as soon as they are formed (two 16-query chunks of
    // 8 values per lane each), which keeps the live set small.
    uint32_t pw[8], sw[8];
    // With a bias, the query part of bias2 (j - i) = bias2 (kj - j0) -
    // bias2 (i - j0) is folded into the staged per-query value (see
    // store_qvals), so log2 P = c s + (bias2 (kj - j0) - staged): two ops.
    const float bias_key = (MOD == kModAdd) ? bias2 * (float)(kj - j0) : 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qo = 8 * g + 4 * h;   // query offset of elements 4g .. 4g + 3
      const f32x4 l4 = *(const f32x4 *)(ls + qo);
      const f32x4 d4 = *(const f32x4 *)(dt + qo);
      // Document masks read the group's ids on every tile and select
      // without a branch: a branch on `full` here doubles the live set of
      // the D = 128 variants and sends K to scratch.
      int4 c4 = int4{0, 0, 0, 0};
      if (DOC) c4 = *(const int4 *)(dc + qo);
      float pr[4], dr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const int i = i0 + qo + e;
        const float x = mod_score<MOD>(s[r], c_log2, bias2, cap_k, cap2, 0.0f, 0.0f);
        float pe = fast_exp2((MOD == kModAdd) ? __builtin_fmaf(s[r], c_log2, bias_key - l4[e])
                                              : log2_p_arg<MOD>(s[r], c_log2, x, l4[e]));
        if (DOC) {
          const int doc_i = (e == 0) ? c4.x : (e == 1) ? c4.y : (e == 2) ? c4.z : c4.w;
          pe = (full || pair_visible<MASK>(a.mask, i, kj, doc_i, doc_j)) ? pe : 0.0f;
        } else if (!full) {
          pe = pair_visible<MASK>(a.mask, i, kj, 0, 0) ? pe : 0.0f;
        }
        pr[e] = pe;
        dr[e] = pe * (dp[r] - d4[e]) * mod_grad<MOD>(x, inv_cap2);
      }
      pw[2 * g] = pack_bf16x2(pr[0], pr[1]);
      pw[2 * g + 1] = pack_bf16x2(pr[2], pr[3]);
      sw[2 * g] = pack_bf16x2(dr[0], dr[1]);
      sw[2 * g + 1] = pack_bf16x2(dr[2], dr[3]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS, 16 queries at a time: the products
    // in order (c, db, dV then dK), each transposed operand read LA products
    // ahead of its use.
    const char *obase0 = ot + rd_tr0, *obase1 = ot + rd_tr1;
    const char *qbase0 = qt_ + rd_tr0, *qbase1 = qt_ + rd_tr1;
    constexpr int NM = 4 * NDB, LA = 2;
    auto rd_op = [&](int m) __attribute__((always_inline)) -> u32x4 {
      const int c = m / (2 * NDB), db = (m >> 1) % NDB;
      const char *b0 = (m & 1) ? qbase0 : obase0, *b1 = (m & 1) ? qbase1 : obase1;
      const s16x4 lo = lds_read_tr(b0 + T::tr_step(c, 0) + 64 * db);
      const s16x4 hi = lds_read_tr(b1 + T::tr_step(c, 1) + 64 * db);
      return u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                   __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
    };
    u32x4 opq[LA + 1];
#pragma unroll
    for (int m = 0; m < LA; ++m) opq[m] = rd_op(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + LA < NM) opq[(m + LA) % (LA + 1)] = rd_op(m + LA);
      __builtin_amdgcn_sched_barrier(0);
      const int c = m / (2 * NDB), db = (m >> 1) % NDB;
      const bf16x8 op = __builtin_bit_cast(bf16x8, opq[m % (LA + 1)]);
      if (m & 1) {
        const bf16x8 sb = __builtin_bit_cast(bf16x8, u32x4{sw[4 * c], sw[4 * c + 1], sw[4 * c + 2], sw[4 * c + 3]});
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, sb, dk[db], 0, 0, 0);
      } else {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]});
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pb, dv[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const Step first{hkv * G, 0};
  // The bias coefficient of the step's query head is carried from the
  // iteration before, as the step's first query and full flag are below:
  // taken where it is needed, its optional table load made the wave wait
  // there for the next tiles' loads as well.  The empty asm keeps the log2
  // scaling at the use.
  float bias_cur = (MOD == kModAdd) ? bias_coeff_uniform(a.score, first.hq, a.Hq) : 0.0f;
  if (n_iter > 0) {
    const int q0f = __builtin_amdgcn_readfirstlane(tile_q0(first.t));
    load_tiles(first, q0f, q_lds0, o_lds0);
    if (wave == 0) store_qvals(fetch_qvals(first, q0f), qv_lse0, qv_dot0, qv_doc0, q0f, bias_cur * kLog2e);
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  // The current step's first query and full flag are carried from the
  // iteration that loaded it, so an iteration looks up one list entry.
  int q0_cur = (n_iter > 0) ? __builtin_amdgcn_readfirstlane(tile_q0(first.t)) : 0;
  bool flag_cur = (n_iter > 0) && tile_flag(first.t);
  // Iteration it (step st): load step it + 1 into the buffers step it - 1
  // used, compute step it, wait for this wave's loads, barrier.
  auto iteration = [&](int it, Step st, char *q_cur, char *o_cur, float *l_cur, float *d_cur,
                       int32_t *c_cur, char *q_nxt, char *o_nxt, float *l_nxt, float *d_nxt,
                       int32_t *c_nxt) __attribute__((always_inline)) {
    const int i0 = q0_cur;
    const bool f0 = flag_cur;
    float b0 = bias_cur;
    if (MOD == kModAdd) asm volatile("" : "+v"(b0));
    QVals nv{INFINITY, 0.0f, -1};
    if (it + 1 < n_iter) {
      const Step nx = next_step(st);
      const int q1 = __builtin_amdgcn_readfirstlane(tile_q0(nx.t));
      q0_cur = q1;
      flag_cur = tile_flag(nx.t);
      load_tiles(nx, q1, q_nxt, o_nxt);
      if (wave == 0) nv = fetch_qvals(nx, q1);
      // The head changes once per n_qt steps, so the slope is recomputed only
      // then (measured 2.7% faster on the GQA window backward); the document
      // variants take it every step, as their registers are full.
      if (MOD == kModAdd && (DOC || nx.hq != st.hq)) bias_cur = bias_coeff_uniform(a.score, nx.hq, a.Hq);
    }
    if (it < n_iter) tile_step(i0, f0, b0 * kLog2e, q_cur, o_cur, l_cur, d_cur, c_cur);
    if (wave == 0 && it + 1 < n_iter) store_qvals(nv, l_nxt, d_nxt, c_nxt, q0_cur, bias_cur * kLog2e);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Steps in pairs; an odd count ends with an empty step (its barrier only),
  // so the step body is built twice, not three times: a third copy pushed
  // the D = 128 document variants over the register budget.
  int it = 0;
  Step st = first;
  for (; it < n_iter; it += 2) {
    iteration(it, st, q_lds0, o_lds0, qv_lse0, qv_dot0, qv_doc0, q_lds1, o_lds1, qv_lse1, qv_dot1, qv_doc1);
    st = next_step(st);
    iteration(it + 1, st, q_lds1, o_lds1, qv_lse1, qv_dot1, qv_doc1, q_lds0, o_lds0, qv_lse0, qv_dot0,
              qv_doc0);
    st = next_step(st);
  }

  // dK = s dX^T Q, dV = P^T dO: lane holds X^T[32 db + 8 g + 4h + e][kj].
  if (kj < a.Skv) {
    float *krow = a.dk + kv_base + (size_t)kj * D;
    float *vrow = a.dv + kv_base + (size_t)kj * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 wk = {dk[db][4 * g + 0] * a.scale, dk[db][4 * g + 1] * a.scale,
                          dk[db][4 * g + 2] * a.scale, dk[db][4 * g + 3] * a.scale};
        const f32x4 wv = {dv[db][4 * g + 0], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
        *(f32x4 *)(krow + 32 * db + 8 * g + 4 * h) = wk;
        *(f32x4 *)(vrow + 32 * db + 8 * g + 4 * h) = wv;
      }
  }
}

template <int D, int MASK, int MOD>
hipError_t launch_main(const BwdArgs &a, hipStream_t stream) {
  const int rows_q = a.gqa_pack ? 32 : kQRows;
  const unsigned grid_q = (unsigned)(((a.Sq + rows_q - 1) / rows_q) * a.B * (a.gqa_pack ? a.Hq / 4 : a.Hq));
  if (grid_q > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, MASK, MOD>), dim3(grid_q), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned grid_k = (unsigned)(((a.Skv + kKRows - 1) / kKRows) * a.B * a.Hkv);
  if (grid_k > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, MASK, MOD>), dim3(grid_k), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D, int MOD>
hipError_t launch_mask(const BwdArgs &a, hipStream_t stream) {
  switch (a.mask.kind) {
    case ATTN_MASK_NONE: return launch_main<D, ATTN_MASK_NONE, MOD>(a, stream);
    case ATTN_MASK_CAUSAL: return launch_main<D, ATTN_MASK_CAUSAL, MOD>(a, stream);
    case ATTN_MASK_SLIDING: return launch_main<D, ATTN_MASK_SLIDING, MOD>(a, stream);
    case ATTN_MASK_PREFIX_LM: return launch_main<D, ATTN_MASK_PREFIX_LM, MOD>(a, stream);
    case ATTN_MASK_DOCUMENT: return launch_main<D, ATTN_MASK_DOCUMENT, MOD>(a, stream);
    case kMaskDocWindow: return launch_main<D, kMaskDocWindow, MOD>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_d(const BwdParams &p, hipStream_t stream) {
  BwdArgs a;
  a.q = (const __bf16 *)p.q;
  a.k = (const __bf16 *)p.k;
  a.v = (const __bf16 *)p.v;
  a.out = (const __bf16 *)p.out;
  a.dout = (const __bf16 *)p.dout;
  a.lse = p.lse;
  a.row_dot = p.row_dot;
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = p.dv;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Skv = p.Skv;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.mask = p.mask;
  a.score = p.score;
  a.bm_num = p.bm_num;
  a.bm_idx = p.bm_idx;
  a.bm_full = p.bm_full;
  a.bm_qnum = p.bm_qnum;
  a.bm_qidx = p.bm_qidx;
  a.bm_qfull = p.bm_qfull;
  a.bm_nqb = p.bm_nqb;
  a.bm_nkb = p.bm_nkb;
  a.bm_batch = p.bm_batch;
  // dQ: grouped heads in fours when the analytic key range applies (a
  // BlockMask row covers 128 query rows).
  a.gqa_pack = (p.bm_num == nullptr && p.Hkv > 0 && (p.Hq / p.Hkv) % 4 == 0) ? 1 : 0;
  if (p.score.kind == ATTN_SCORE_SOFTCAP) return launch_mask<D, kModCap>(a, stream);
  if (p.score.kind == ATTN_SCORE_NONE) return launch_mask<D, kModRaw>(a, stream);
  return launch_mask<D, kModAdd>(a, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams &p, hipStream_t stream) {
  if (p.D == 64) return launch_d<64>(p, stream);
  if (p.D == 128) return launch_d<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
