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
//    consecutive rows.  With grouped heads (Hq / Hkv a multiple of 4, no
//    BlockMask) the 128 rows are 32 positions of four heads sharing a kv
//    head, one head per wave, so all four waves need the same key tiles.
//    Key tiles of 64 rows (128 for unmasked D=64).  Two workgroups per CU,
//    so each SIMD interleaves two waves: one's MFMAs run beside the other's
//    softmax.
//  * Scores are computed transposed, S^T = K·Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand, Q^T (kept in
//    VGPRs for the whole kernel) the B operand.  In the 32x32 accumulator
//    layout a lane then holds one query column and 16 keys, so the row max
//    and row sum of the softmax are in-lane reductions plus one exchange
//    between the two 32-lane halves (v_permlane32_swap).
//  * P^T leaves the accumulator already in the B-operand layout of the next
//    MFMA, O^T += V^T·P^T, with the key order inside each 16-key chunk
//    permuted identically on both operands; V^T fragments are read from the
//    row-major V tile with ds_read_b64_tr_b16 (the gfx950 transposing LDS
//    read), so V is never transposed in memory.
//  * Software pipeline inside each wave: the S MFMAs of key tile n+1 are
//    issued before the softmax of tile n, so the matrix cores work while the
//    VALU computes exp2; K is staged one tile ahead of V.
//  * K/V tiles move HBM/L2 -> LDS with buffer_load ... lds (no VGPR staging,
//    rows past Skv read as zero).  A tile is stored as 1 KiB blocks of rows:
//    key k lives in block k mod NB at slot k / NB, blocks padded apart, so
//    both the 16-byte K reads and the transposed V reads of a wave hit
//    distinct banks and every LDS address is a per-lane base plus a
//    compile-time offset.  The double buffers are four separate LDS
//    objects named at every access (the tile loop is unrolled by two), so
//    the compiler sees that reading one buffer does not wait on loads still
//    landing in another: each wave waits for its loads only at the barrier
//    that ends the iteration.
//  * The softmax tail of a tile (exp2, P·V, next S) and the issue of the
//    tile loads run at raised wave priority (s_setprio), so the matrix-core
//    work and the loads of one wave issue ahead of the other wave's max
//    reductions.
//  * exp2 with scale·log2(e) folded into one FMA; the running max is raised
//    only when a tile exceeds it by a margin; key tiles are visited last to
//    first, so under causal-type masks and ALiBi the first tile already
//    holds the row's largest scores; LSE in natural log on output.
//  * The 8 XCDs (each with its own L2) take workgroups round-robin; the head
//    index is permuted so that each XCD works on a contiguous run of heads,
//    and the query heads of a GQA group read their K/V through one L2.
//  * Causal-type masks: workgroups with the most key tiles are launched
//    first (with a BlockMask, the query tiles with the most listed blocks,
//    ranked by each wave in registers); waves skip tiles that hold no
//    visible key for their rows and skip the predicate on tiles where every
//    key is visible.
//  * The bf16 output leaves through LDS: each wave stages its rows in a
//    free tile buffer and stores whole rows, 16 bytes per lane.
#include <type_traits>

#include "kernels.h"

namespace attn {
namespace {

constexpr int kBM = 128;       // query rows per workgroup
// BlockMask blocks on this path are 128 keys wide (host-checked).
constexpr int kMaskBlock = 128;
constexpr int kThreads = 256;  // 4 waves
constexpr int kListCap = 1024; // BlockMask entries staged in LDS per query tile (host-checked)
// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;
constexpr int kKPad = 16;      // bytes between K row blocks
constexpr int kVPad = 64;      // bytes between V row blocks

// D and the key-tile length BN: 128 at D = 64 without a mask, where the
// per-tile fixed work (loads, max, barrier) would otherwise weigh on only 16
// MFMAs (measured +6% on dense D = 64; under causal-type masks the longer
// tiles lose more on the diagonal than they gain, so those keep 64).
template <int D, int BN_>
struct FwdCfg {
  static constexpr int BN = BN_;                  // key rows per tile
  static constexpr int KB = BN / 32;              // 32-key blocks of S^T per tile
  static constexpr int NCH = BN / 16;             // 16-key chunks of P per tile
  static constexpr int TPB = kMaskBlock / BN;     // tiles per BlockMask block
  static constexpr int TPB_SHIFT = TPB == 2 ? 1 : 0;
  static_assert(TPB == 1 << TPB_SHIFT, "tile -> block is a shift");
  static constexpr int ROWB = D * 2;              // bytes of one K/V row
  static constexpr int NB = BN * ROWB / 1024;     // 1 KiB row blocks per tile (8 or 16)
  static constexpr int KBLK = 1024 + kKPad;
  static constexpr int VBLK = 1024 + kVPad;
  static constexpr int KTILE = NB * KBLK;         // bytes
  static constexpr int VTILE = NB * VBLK;
  static constexpr int NDC = D / 16;              // 16-wide d chunks of S^T = K Q^T
  static constexpr int NDB = D / 32;              // 32-row d blocks of O^T
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int LOADS = NB / 4;            // direct loads per wave per tile (K or V)
  static_assert(NB % 4 == 0 && 32 % NB == 0, "block mapping");
};

struct KernelArgs {
  const __bf16 *q, *k, *v;
  void *out;           // bf16 or fp32 [B, Hq, Sq, D]
  float *lse;
  int B, Hq, Hkv, Sq, Skv;
  int n_qtiles;        // query tiles per (b, head unit): ceil(Sq / rows per workgroup)
  int gqa_pack;        // 1: a workgroup is 32 positions of four query heads (see the kernel)
  float scale_log2;    // scale * log2(e)
  MaskArgs mask;
  ScoreArgs score;
  const int32_t *bm_num, *bm_idx;
  const uint8_t *bm_full;
  int bm_nqb, bm_nkb, bm_batch;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ s16x4 lds_read_tr(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}

// How the log2-domain score x is formed from the dot product s:
//  kModRaw   x = c s, never materialised: the row max is taken on the raw dot
//            products (c > 0 preserves order) and p = 2^(c s - m) is one FMA
//            and one exp2;
//  kModBias  x = c s + bias, materialised before the max (any bias, or a
//            scale <= 0);
//  kModCap   x = C tanh(c s / C), the soft cap, materialised before the max;
//  kModLin   x = c s + a (j - i), a bias linear in the key-query distance
//            (ALiBi, relative position) with c > 0, never materialised: the
//            part a * (offset of the element within its 32-key block) / c is
//            the C input of the first S MFMA of every block (a constant
//            register block), so the accumulator holds s + that, and the
//            per-lane remainder a (block's first key - i) joins the exp2's
//            addend and the max as one value per block.  The ALiBi path then
//            costs the raw path's VALU work per score.
constexpr int kModRaw = 0, kModBias = 1, kModCap = 2, kModLin = 3;

// Compile-time variants: D, the mask kind, the score form MOD and the output
// dtype.
template <int D, int MASK, int MOD, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(KernelArgs a) {
  constexpr bool GEN = MOD == kModBias || MOD == kModCap;   // x materialised before the max
  constexpr bool LIN = MOD == kModLin;
  // Mask terms: document ids compared (DOCUMENT, and DOCUMENT with a window)
  // and a window on i - j (SLIDING, and DOCUMENT with a window).
  constexpr bool DOC = MASK == ATTN_MASK_DOCUMENT || MASK == kMaskDocWindow;
  constexpr bool WIN = MASK == ATTN_MASK_SLIDING || MASK == kMaskDocWindow;
  using C = FwdCfg<D, (D == 64 && MASK == ATTN_MASK_NONE) ? 128 : 64>;
  constexpr int kBN = C::BN;
  static_assert(!DOC || kBN == 64, "document ids are staged one per lane");
  // K and V double buffers as four distinct LDS objects, always addressed
  // through their own names: the compiler can then tell that reading one
  // buffer does not depend on buffer->LDS loads still in flight to another,
  // and does not wait for them (the barriers below order the buffers).
  __shared__ __align__(16) char k_lds0[C::KTILE];
  __shared__ __align__(16) char k_lds1[C::KTILE];
  __shared__ __align__(16) char v_lds0[C::VTILE];
  __shared__ __align__(16) char v_lds1[C::VTILE];
  __shared__ __align__(16) int32_t kdoc[3][64];    // document ids of staged key tiles (BN = 64)
  __shared__ int32_t kdoc_mm[3][2];                // their min and max
  __shared__ __align__(16) int32_t s_blk[kListCap];
  __shared__ uint8_t s_full[kListCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;   // kept per-lane: branches on it stay exec-masked, which keeps the schedule tight
  // The same index in a scalar register, for the tile loads' LDS
  // destinations (M0 takes a scalar; computed from the per-lane index they
  // would hold a vector register each).
  const int wave_s = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;      // lane half: selects keys 4h..4h+3 of each 8
  const int l32 = lane & 31;    // query column of this lane

  // What a workgroup covers.  By default one query head and 128 consecutive
  // query rows, wave w taking rows 32w .. 32w + 31.  With gqa_pack (grouped
  // heads, Hq / Hkv a multiple of 4, no BlockMask) it covers 32 query
  // positions of four query heads that share a kv head, wave w taking head
  // 4g + w: every wave then needs the same key tiles, so the workgroup visits
  // the key range of 32 rows instead of the union of four staggered ones (a
  // 1024-key window spans 17 tiles of 64 keys instead of 18), and no wave
  // sits out a tile its neighbours compute.
  // Workgroups go round-robin to the 8 XCDs; each XCD gets a contiguous run
  // of head units, so the query heads of one kv head share an L2.
  const int pack = a.gqa_pack;
  const int hunits = pack ? a.Hq / 4 : a.Hq;   // head units per batch row
  const int bh_count = a.B * hunits;
  const int xh = (int)(blockIdx.x % bh_count);
  const int bh = (bh_count % 8 == 0) ? (xh % 8) * (bh_count / 8) + xh / 8 : xh;
  const int b = bh / hunits;
  const int hu = bh - b * hunits;
  const int hq = pack ? 4 * hu + wave_s : hu;   // wave-uniform
  // Heaviest query tiles first.  Without a BlockMask the later tiles are the
  // heavier ones (causal-type masks give them more keys).  With one, a tile's
  // work is its listed block count, which need not grow with the tile index
  // (documents): every wave ranks the tiles of its batch row by count
  // (descending; ties, the later tile first) and takes the tile at its
  // workgroup's dispatch position.
  const int pos = (int)(blockIdx.x / bh_count);
  int qt = a.n_qtiles - 1 - pos;
  int n_ranked = -1;   // the tile's clamped list length, when the ranking ran
  if (a.bm_num && a.n_qtiles <= kOrderCap) {
    const int bb = (a.bm_batch == 1) ? 0 : b;
    qt = work_ordered_tile(a.bm_num + (size_t)bb * a.bm_nqb, a.n_qtiles, min(a.bm_nkb, kListCap), pos,
                           true, &n_ranked);
  }
  const int hkv = (hq * a.Hkv) / a.Hq;
  const int rows = pack ? 32 : kBM;   // query positions per workgroup
  const int q0 = qt * rows;
  const int qw0 = pack ? q0 : q0 + wave * 32;
  const int qw1 = min(qw0 + 31, a.Sq - 1);
  const int qi = qw0 + l32;

  const size_t q_base = ((size_t)(b * a.Hq + hq) * a.Sq) * D;
  const size_t kv_base = ((size_t)(b * a.Hkv + hkv) * a.Skv) * D;
  // The row's document id is fetched now, so its latency overlaps the
  // BlockMask list's (it is waited for after the list is staged).
  const int32_t *doc_row = DOC ? a.mask.doc_ids + (size_t)b * a.mask.doc_stride : nullptr;
  const int doc_i = DOC ? doc_row[min(qi, a.Sq - 1)] : 0;

  // Q^T fragments: lane holds Q[qi][16c + 8h .. 16c + 8h + 7] (rows past Sq
  // read row Sq-1 and are never stored).  Loaded in the prologue, after the
  // first tile loads are issued, so the two latencies overlap.
  bf16x8 qf[C::NDC];
  const bf16x8 *q_src = (const bf16x8 *)(a.q + q_base + (size_t)min(qi, a.Sq - 1) * D);
#pragma unroll
  for (int c = 0; c < C::NDC; ++c) qf[c] = q_src[2 * c + h];

  // ---- key tiles to visit.  A BlockMask row is staged in LDS so the tile
  // loop reads it without vector memory waits (the host limits a row to
  // kListCap entries).
  const int qlast = min(q0 + rows, a.Sq) - 1;
  int n_tiles;
  int t_first = 0;
  const int32_t *bm_list = nullptr;
  const uint8_t *bm_flags = nullptr;
  if (a.bm_num) {
    const int bb = (a.bm_batch == 1) ? 0 : b;
    const size_t row = (size_t)bb * a.bm_nqb + qt;
    // Counts and indices are device data: clamp them so a malformed list
    // can only drop tiles, never address outside K/V.
    int n_blocks = __builtin_amdgcn_readfirstlane(n_ranked);
    if (n_blocks < 0) n_blocks = min(max(a.bm_num[row], 0), min(a.bm_nkb, kListCap));
    n_tiles = n_blocks * C::TPB;
    bm_list = a.bm_idx + row * a.bm_nkb;
    if (a.bm_full) bm_flags = a.bm_full + row * a.bm_nkb;
    // The row's loads share one memory latency with the Q and document-id
    // loads issued above.
    stage_list_row<kListCap, kThreads>(bm_list, bm_flags, n_blocks, s_blk, s_full, tid);
    __syncthreads();   // the list is read by every wave from here on
  } else {
    int lo = 0, hi = a.Skv;
    if (MASK == ATTN_MASK_CAUSAL || MASK == ATTN_MASK_DOCUMENT) {
      hi = min(a.Skv, qlast + 1);
    } else if (WIN) {
      hi = min(a.Skv, qlast + 1);
      lo = max(0, q0 - a.mask.window + 1);
    } else if (MASK == ATTN_MASK_PREFIX_LM) {
      hi = min(a.Skv, max(qlast + 1, a.mask.prefix_len));
    }
    t_first = lo / kBN;
    n_tiles = (hi > lo) ? (hi + kBN - 1) / kBN - t_first : 0;
  }
  // Key tiles are visited from the last to the first: under causal-type
  // masks the first one visited is the diagonal, and with a bias that grows
  // with the key index (ALiBi) it carries the row's largest scores, so the
  // running max is set early and rarely raised afterwards.
  auto tile_key0 = [&](int n) __attribute__((always_inline)) -> int {
    n = n_tiles - 1 - n;
    if (bm_list) {
      const int bi = n >> C::TPB_SHIFT;   // n >= 0
      const int blk = s_blk[bi];   // bi < n_blocks <= kListCap
      if (blk < 0 || blk >= a.bm_nkb) return a.Skv;      // treated as an empty tile
      return blk * kMaskBlock + (n & (C::TPB - 1)) * kBN;
    }
    return (t_first + n) * kBN;
  };
  auto tile_block_full = [&](int n) __attribute__((always_inline)) -> bool {
    n = n_tiles - 1 - n;
    if (!bm_flags) return false;
    const int bi = n >> C::TPB_SHIFT;
    return s_full[bi] != 0;
  };

  // ---- HBM/L2 -> LDS through buffer_load ... lds.  Wave w, load i fills
  // row block blk = 4i + w: lane L writes bytes [16L, 16L + 16) of the block,
  // i.e. slot L / CPR (key blk + NB * slot), 16-byte chunk L % CPR.  Keys
  // past Skv fall outside the buffer's range and read as zero.
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.k + kv_base), (short)0, a.Skv * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.v + kv_base), (short)0, a.Skv * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t d_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(doc_row ? doc_row : a.mask.doc_ids), (short)0, doc_row ? a.Skv * 4 : 0, kBufferFlags);
  // Byte offset of this lane's chunk for load i = 0; load i is 4 rows
  // further on, which goes into the scalar offset with the tile's own.  key0
  // is wave-uniform; on the BlockMask path it comes from LDS, so it is moved
  // to a scalar register explicitly.
  const int ld_off = ((wave + C::NB * (lane / C::CPR)) * D + (lane % C::CPR) * 8) * 2;
  auto load_k = [&](char *dst, int key0) __attribute__((always_inline)) {
    const int soff = __builtin_amdgcn_readfirstlane(key0 * D * 2);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (lds_void *)(dst + (4 * i + wave_s) * C::KBLK), 16,
                                               ld_off, soff + i * (4 * D * 2), 0, 0);
  };
  auto load_v = [&](char *dst, int key0) __attribute__((always_inline)) {
    const int soff = __builtin_amdgcn_readfirstlane(key0 * D * 2);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rsrc, (lds_void *)(dst + (4 * i + wave_s) * C::VBLK), 16,
                                               ld_off, soff + i * (4 * D * 2), 0, 0);
  };
  // Document ids of a key tile go through wave 0's registers into kdoc (a
  // plain LDS store, so later reads of kdoc never wait for the buffer->LDS
  // loads): fetched at the start of an iteration, stored at its end.
  auto load_doc = [&](int key0) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_raw_buffer_load_b32(d_rsrc, lane * 4, __builtin_amdgcn_readfirstlane(key0 * 4), 0);
  };

  // Per-lane LDS read bases.  K (A operand of S^T): key kb*32 + l32, bytes
  // of chunk 2c + h.  V^T (ds_read_b64_tr_b16): within each 16-lane group,
  // lanes 4r..4r+3 point at 4 consecutive d of key 4h + r (+16c, +8 for the
  // second read); the read hands lane i the 4 keys' values at d = i.
  // Key kk + x with x = the lane's part lives at block (kk % NB) + x % NB:
  // the compile-time parts below never carry (kk % NB + x < NB).
  const int k_rd = (l32 % C::NB) * C::KBLK + (l32 / C::NB) * C::ROWB + h * 16;
  const int tr_j = lane & 15;
  const int tr_key = 4 * h + (tr_j >> 2);
  const int v_rd = tr_key * C::VBLK + (16 * ((lane >> 4) & 1) + 4 * (tr_j & 3)) * 2;
  constexpr auto v_key_off = [](int kk) { return (kk % C::NB) * C::VBLK + (kk / C::NB) * C::ROWB; };

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
  const float bias2 = (MOD == kModBias || LIN) ? bias_coeff(a.score, hq, a.Hq) * kLog2e : 0.0f;
  // kModLin: C input of each 32-key block's first S MFMA, element r being key
  // 8 (r / 4) + r % 4 of the block (past the lane's 4h), scaled by 1 / c.
  f32x16 c_lin;
  if constexpr (LIN) {
    const float bc = bias2 / c_log2;
#pragma unroll
    for (int r = 0; r < 16; ++r) c_lin[r] = bc * (float)(8 * (r >> 2) + (r & 3));
  }
  // Soft cap in log2 units and its exponent factor (2 / cap) * c.
  const float cap2 = (MOD == kModCap) ? a.score.softcap * kLog2e : 0.0f;
  const float cap_k = (MOD == kModCap) ? (2.0f / a.score.softcap) * c_log2 : 0.0f;
  asm volatile("" ::"v"(doc_i));   // complete the load before the tile loop
  // Range of the wave's row ids (rows past Sq repeat row Sq - 1): a key tile
  // whose id range misses it holds no visible key for the wave, and one
  // whose ids and the rows' are all one id is visible wherever causality
  // allows.  Neither test assumes sorted ids.
  const int dmin_w = DOC ? wave_min_i32(doc_i) : 0;
  const int dmax_w = DOC ? wave_max_i32(doc_i) : 0;
  // Wave 0 stages a tile's ids (one per lane) with their min and max.
  auto store_doc = [&](int slot, int id) __attribute__((always_inline)) {
    kdoc[slot][lane] = id;
    const int mn = wave_min_i32(id), mx = wave_max_i32(id);
    if (lane == 0) {
      kdoc_mm[slot][0] = mn;
      kdoc_mm[slot][1] = mx;
    }
  };

  // Visibility class of a key tile for this wave (dslot: the tile's slot of
  // staged document ids).
  auto tile_empty = [&](int k0, int dslot) __attribute__((always_inline)) -> bool {
    bool e = (qw0 >= a.Sq) || (k0 >= a.Skv);
    if (MASK == ATTN_MASK_CAUSAL || MASK == ATTN_MASK_DOCUMENT) e = e || (k0 > qw1);
    if (WIN) e = e || (k0 > qw1) || (qw0 - (k0 + kBN - 1) >= a.mask.window);
    if (MASK == ATTN_MASK_PREFIX_LM) e = e || ((k0 > qw1) && (k0 >= a.mask.prefix_len));
    if (DOC) e = e || (kdoc_mm[dslot][1] < dmin_w) || (kdoc_mm[dslot][0] > dmax_w);
    return e;
  };
  auto doc_one_id = [&](int dslot) __attribute__((always_inline)) -> bool {
    return kdoc_mm[dslot][0] == kdoc_mm[dslot][1] && dmin_w == dmax_w && kdoc_mm[dslot][0] == dmin_w;
  };
  auto tile_full = [&](int k0, int n, int dslot) __attribute__((always_inline)) -> bool {
    bool f = (k0 + kBN <= a.Skv);
    if (MASK == ATTN_MASK_CAUSAL) f = f && (k0 + kBN - 1 <= qw0);
    if (MASK == ATTN_MASK_DOCUMENT)
      f = f && (k0 + kBN - 1 <= qw0) && (tile_block_full(n) || doc_one_id(dslot));
    if (MASK == ATTN_MASK_SLIDING) f = f && (k0 + kBN - 1 <= qw0) && (qw1 - k0 < a.mask.window);
    if (MASK == kMaskDocWindow)
      f = f && (k0 + kBN - 1 <= qw0) && (qw1 - k0 < a.mask.window) &&
          (tile_block_full(n) || doc_one_id(dslot));
    if (MASK == ATTN_MASK_PREFIX_LM) f = f && ((k0 + kBN - 1 <= qw0) || (k0 + kBN <= a.mask.prefix_len));
    return f;
  };

  // Initial accumulator of an S block: zero, or the kModLin bias part.
  auto s_init = [&]() __attribute__((always_inline)) -> f32x16 {
    if constexpr (LIN) return c_lin;
    else return f32x16{};
  };
  // S^T = K Q^T for the two 32-key blocks of the K tile at kt.
  auto compute_s = [&](f32x16 (&s)[C::KB], const char *kt) __attribute__((always_inline)) {
    const char *kbase = kt + k_rd;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
      for (int c = 0; c < C::NDC; ++c) {
        const bf16x8 ka = *(const bf16x8 *)(kbase + (32 * kb / C::NB) * C::ROWB + 32 * c);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], c > 0 ? s[kb] : s_init(), 0, 0, 0);
      }
    }
  };

  // Head of the softmax of one tile (scores s, first key k0, index n): bias,
  // mask, tile max, threshold rescale of O and l.  Returns the exp2 addend of
  // each 32-key block: p = 2^(x - mu) is 2^(s + add) on the materialised
  // forms and 2^(c s + add) on the others (add = -mu, and for kModLin the
  // block's bias remainder too).
  auto softmax_head = [&](f32x16 (&s)[C::KB], int k0, int n, int dslot, float (&add)[C::KB])
                          __attribute__((always_inline)) {
    const bool full = tile_full(k0, n, dslot);
    // Accumulator element r of block kb is key j = jb + kb*32 + 8(r/4) + r%4
    // with jb = k0 + 4h.
    const int jb = k0 + 4 * h;
    if constexpr (MOD == kModBias) {
      const float cb = bias2 * (float)(jb - qi);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float off = (float)(kb * 32 + 8 * (r >> 2) + (r & 3));
          s[kb][r] = __builtin_fmaf(s[kb][r], c_log2, __builtin_fmaf(bias2, off, cb));
        }
    } else if constexpr (MOD == kModCap) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = softcap_log2_fast(s[kb][r], cap_k, cap2);
    }
    if (!full && !DOC) {
      // Partial tile, masks of positions only: every kind's visible keys of
      // a row form one interval of offsets, lo <= off <= hi (CAUSAL and
      // SLIDING end at the diagonal, PREFIX_LM at the later of the diagonal
      // and the prefix end, and all at the last key; SLIDING starts W - 1
      // keys before the diagonal), tested as one unsigned compare per
      // element: (hi - off) < (hi - lo + 1).  -inf where hidden (for the
      // raw scores too: c > 0 on that path).
      const int dq = qi - jb;                       // j <= qi  <=>  off <= dq
      int hi = a.Skv - jb - 1;
      int lo = 0;
      if (MASK == ATTN_MASK_CAUSAL || WIN) hi = min(hi, dq);
      if (MASK == ATTN_MASK_PREFIX_LM) hi = min(hi, max(dq, a.mask.prefix_len - jb - 1));
      if (WIN) lo = dq - a.mask.window + 1;
      const unsigned span = (hi >= lo) ? (unsigned)(hi - lo) + 1u : 0u;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          if constexpr (WIN) s[kb][r] = ((unsigned)(hi - off) < span) ? s[kb][r] : -INFINITY;
          else s[kb][r] = (off <= hi) ? s[kb][r] : -INFINITY;   // lo = 0: one compare with a constant
        }
    }
    if (!full && DOC) {
      // Partial tile under a document mask: the predicate per element,
      // with the key ids staged in LDS.
      const int dq = qi - jb;                       // j <= qi  <=>  off <= dq
      int32_t kd[C::KB][4][4];
      if (DOC) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int4 t = *(const int4 *)&kdoc[dslot][kb * 32 + 8 * g + 4 * h];
            kd[kb][g][0] = t.x; kd[kb][g][1] = t.y; kd[kb][g][2] = t.z; kd[kb][g][3] = t.w;
          }
      }
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          bool vis = off < a.Skv - jb;
          if (MASK == ATTN_MASK_CAUSAL) vis = vis && (off <= dq);
          if (MASK == ATTN_MASK_SLIDING) vis = vis && (off <= dq) && (dq - off < a.mask.window);
          if (MASK == ATTN_MASK_PREFIX_LM) vis = vis && ((off <= dq) || (off < a.mask.prefix_len - jb));
          if (MASK == ATTN_MASK_DOCUMENT) vis = vis && (off <= dq) && (kd[kb][r >> 2][r & 3] == doc_i);
          if (MASK == kMaskDocWindow)
            vis = vis && (off <= dq) && (dq - off < a.mask.window) && (kd[kb][r >> 2][r & 3] == doc_i);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }

    // Tile row max (raw or modified scores), shared by the two halves.  Four
    // independent partial maxima keep the dependency chain short; two per
    // 32-key block (kModLin adds each block's bias remainder after the max).
    float mx[2 * C::KB];
#pragma unroll
    for (int i = 0; i < 2 * C::KB; ++i) mx[i] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        // One v_max3 folds two scores into a partial max (the compiler's own
        // tree used 24 max ops for 32 scores; this is 16): +2-3% on causal
        // and soft-cap D=64, neutral elsewhere, same results.
        float &m = mx[2 * kb + ((r >> 1) & 1)];
        asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(m), "v"(s[kb][r]), "v"(s[kb][r + 1]));
      }
    // kModLin: the bias of element r of block kb is bias2 (jb + 32 kb - qi)
    // plus the part already in the accumulator.
    float lin[C::KB];
    lin[0] = LIN ? bias2 * (float)(jb - qi) : 0.0f;
#pragma unroll
    for (int kb = 1; kb < C::KB; ++kb) lin[kb] = LIN ? __builtin_fmaf(bias2, 32.0f * kb, lin[0]) : 0.0f;
    float tmax = -INFINITY;
    if constexpr (LIN) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
        tmax = __builtin_fmaxf(tmax, __builtin_fmaf(__builtin_fmaxf(mx[2 * kb], mx[2 * kb + 1]), c_log2, lin[kb]));
    } else {
#pragma unroll
      for (int kb = 0; kb < C::KB; kb += 2)
        tmax = __builtin_fmaxf(tmax, __builtin_fmaxf(__builtin_fmaxf(mx[2 * kb], mx[2 * kb + 1]),
                                                     __builtin_fmaxf(mx[2 * kb + 2], mx[2 * kb + 3])));
      if constexpr (!GEN) tmax *= c_log2;
    }
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
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) add[kb] = lin[kb] - mu;
  };

  // Tail of the softmax: P = 2^(x - mu) and O^T += V^T P^T (V in buffer
  // tile vt), one 16-key chunk at a time, each chunk's P·V MFMAs right after its
  // exp2s.  With WITH_S the S MFMAs of the next tile (K tile kt) are
  // spread over the chunks: one straight-line region in which the matrix
  // cores and the VALU work side by side.  LDS reads are issued ahead of
  // their use, each chunk's V fragments at its start and the K fragments a
  // whole chunk early, and scheduling barriers keep the compiler from
  // sinking them back next to their MFMAs (measured 4-8% faster than reads
  // placed by the scheduler).
  auto softmax_tail = [&](auto with_s, f32x16 (&s)[C::KB], const float (&add)[C::KB], const char *vt,
                          f32x16 (&sn)[C::KB], const char *kt) __attribute__((always_inline)) {
    constexpr bool WITH_S = decltype(with_s)::value;
    constexpr int S_PER_CHUNK = C::KB * C::NDC / C::NCH;   // S MFMAs per 16-key chunk
    const char *vbase = vt + v_rd;
    const char *kbase = kt + k_rd;
    float ps[4];   // independent partial row sums, seeded by the first chunk
    // K fragment i of the next tile's S MFMAs (block i / NDC, d chunk i % NDC).
    auto k_frag = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      const int kb = i / C::NDC, cc = i % C::NDC;
      return *(const bf16x8 *)(kbase + (32 * kb / C::NB) * C::ROWB + 32 * cc);
    };
    bf16x8 kf[2][S_PER_CHUNK];   // this chunk's K fragments and the next chunk's
    if constexpr (WITH_S) {
#pragma unroll
      for (int t = 0; t < S_PER_CHUNK; ++t) kf[0][t] = k_frag(t);
    }
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      // Reads first: the next chunk's K fragments and this chunk's V^T.
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (WITH_S) {
        if (c + 1 < C::NCH) {
#pragma unroll
          for (int t = 0; t < S_PER_CHUNK; ++t) kf[(c + 1) & 1][t] = k_frag((c + 1) * S_PER_CHUNK + t);
        }
      }
      s16x4 vlo[C::NDB], vhi[C::NDB];
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        vlo[db] = lds_read_tr(vbase + v_key_off(16 * c) + 64 * db);
        vhi[db] = lds_read_tr(vbase + v_key_off(16 * c + 8) + 64 * db);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (WITH_S) {
#pragma unroll
        for (int t = 0; t < S_PER_CHUNK; ++t) {
          const int i = c * S_PER_CHUNK + t;
          const int kb = i / C::NDC, cc = i % C::NDC;
          sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c & 1][t], qf[cc], cc == 0 ? s_init() : sn[kb],
                                                           0, 0, 0);
        }
      }
      const int kb = c >> 1;
      const int r0 = 8 * (c & 1);
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float p0, p1;
        if constexpr (GEN) {
          p0 = fast_exp2(s[kb][r0 + e] + add[kb]);
          p1 = fast_exp2(s[kb][r0 + e + 1] + add[kb]);
        } else {
          p0 = fast_exp2(__builtin_fmaf(s[kb][r0 + e], c_log2, add[kb]));
          p1 = fast_exp2(__builtin_fmaf(s[kb][r0 + e + 1], c_log2, add[kb]));
        }
        // The first chunk seeds the partial sums rather than adding to zero
        // (0 + x is not folded away: it could change the sign of a zero).
        if (c == 0) ps[e >> 1] = p0 + p1; else ps[e >> 1] += p0 + p1;
        pw[e >> 1] = pack_bf16x2(p0, p1);
      }
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      // The sums are formed here, so the chunk's fp32 p values die with it
      // instead of staying live until the end of the tile.
      asm volatile("" : "+v"(ps[0]), "+v"(ps[1]), "+v"(ps[2]), "+v"(ps[3]));
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const s16x4 lo = vlo[db];
        const s16x4 hi = vhi[db];
        const u32x4 vw = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pb,
                                                        o[db], 0, 0, 0);
      }
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };

  // ---- prologue: K0, V0, K1 (and the document ids of tiles 0, 1)
  // resident; S0 computed.  Tile n uses K and V buffer n % 2 and document
  // slot n % 3.
  f32x16 sa[C::KB], sb[C::KB];
  if (n_tiles > 0) {
    // The document ids go first: their stores then wait for them alone,
    // not for the tile loads issued after them.
    int d0 = 0, d1 = 0;
    if (DOC && wave == 0) {
      d0 = load_doc(tile_key0(0));
      if (n_tiles > 1) d1 = load_doc(tile_key0(1));
    }
    load_k(k_lds0, tile_key0(0));
    load_v(v_lds0, tile_key0(0));
    if (n_tiles > 1) load_k(k_lds1, tile_key0(1));
    if (DOC && wave == 0) {
      store_doc(0, d0);
      if (n_tiles > 1) store_doc(1, d1);
    }
  }
  // The empty asm statements make the Q loads complete here, so the tile
  // loop never waits on them.
#pragma unroll
  for (int c = 0; c < C::NDC; ++c) asm volatile("" ::"v"(qf[c]));
  if (n_tiles > 0) __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) expcnt(0) lgkmcnt(0)
  __syncthreads();
  // The first key and liveness of the current tile and the first key of the
  // next are carried from one iteration to the next, so an iteration reads
  // one new list entry (BlockMask) and classifies one new tile.
  int key_cur = (n_tiles > 0) ? __builtin_amdgcn_readfirstlane(tile_key0(0)) : 0;
  int key_nxt = (n_tiles > 1) ? __builtin_amdgcn_readfirstlane(tile_key0(1)) : 0;
  bool live_cur = (n_tiles > 0) && !tile_empty(key_cur, 0);
  if (live_cur) compute_s(sa, k_lds0);
  // Iteration 0 refills K buffer 0 (tile 2): every wave must be done reading
  // tile 0 from it first.  Later refills target a buffer last read before
  // the previous iteration's barrier.
  __syncthreads();

  // ---- tile loop, unrolled by two so that the S accumulators alternate and
  // every LDS access names its buffer.
  // Iteration n: (1) start loading K[n+2] and V[n+1] into the buffers tile
  // n-1 freed (k_fill, v_fill) and fetch the document ids of tile n+2;
  // (2) softmax of tile n with its P·V MFMAs (V tile v_cur), interleaved with
  // the S MFMAs of tile n+1 (K tile k_next); (3) store the ids into the slot
  // tile n-1 freed, wait for this wave's loads, barrier.
  auto iteration = [&](int n, f32x16 (&s_cur)[C::KB], f32x16 (&s_next)[C::KB], char *k_fill, char *v_fill,
                       const char *v_cur, const char *k_next) __attribute__((always_inline)) {
    const int k0 = key_cur;
    const int k2 = (n + 2 < n_tiles) ? __builtin_amdgcn_readfirstlane(tile_key0(n + 2)) : 0;
    int doc_fill = 0;
    // The loads issue at raised priority too (measured 1-3% faster): only
    // the softmax head runs at the base priority.
    __builtin_amdgcn_s_setprio(1);
    if (n + 2 < n_tiles) {
      if (DOC && wave == 0) doc_fill = load_doc(k2);
      load_k(k_fill, k2);
    }
    if (n + 1 < n_tiles) load_v(v_fill, key_nxt);
    __builtin_amdgcn_s_setprio(0);
    const bool cur_live = live_cur;
    const bool next_live = (n + 1 < n_tiles) && !tile_empty(key_nxt, (n + 1) % 3);
    live_cur = next_live;
    key_cur = key_nxt;
    key_nxt = k2;
    if (cur_live) {
      // The next tile's S is computed whether or not that tile is live for
      // this wave (a dead or absent tile reads a stale, valid K buffer and
      // the result is never used): one code path keeps the whole tail in a
      // single scheduling region.
      float add[C::KB];
      softmax_head(s_cur, k0, n, n % 3, add);
      // The tail (exp2, P·V and the next tile's S on the matrix cores) runs
      // at raised wave priority, so a wave there issues ahead of waves in
      // their softmax head or waiting on loads: measured 6-7% faster on
      // causal and 4-5% on the GQA window workload, dense unchanged.
      __builtin_amdgcn_s_setprio(1);
      softmax_tail(std::true_type{}, s_cur, add, v_cur, s_next, k_next);
      __builtin_amdgcn_s_setprio(0);
    } else if (next_live) {
      compute_s(s_next, k_next);
    }
    if (DOC && wave == 0 && n + 2 < n_tiles) store_doc((n + 2) % 3, doc_fill);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads and LDS stores are done
    __syncthreads();
  };
  int n = 0;
  for (; n + 1 < n_tiles; n += 2) {
    iteration(n, sa, sb, k_lds0, v_lds1, v_lds0, k_lds1);
    iteration(n + 1, sb, sa, k_lds1, v_lds0, v_lds1, k_lds0);
  }
  if (n < n_tiles) iteration(n, sa, sb, k_lds0, v_lds1, v_lds0, k_lds1);

  // ---- epilogue: O / l, LSE = (m + log2 l) ln 2.
  const float l_tot = half_swap_sum(l_run);
  const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  if constexpr (!OUT_F32) {
    // The bf16 rows go out through LDS: each wave stages its 32 rows in one
    // of the four tile buffers (free once the loop's last barrier has
    // passed: every wave is done reading them and no load into them is in
    // flight), then each store writes whole 16-byte chunks of 64 / (D / 8)
    // full rows, 8 (D = 128) or 4 (D = 64) stores per lane instead of 16 or
    // 8 scattered 8-byte ones.  The staging row stride of D * 2 + 16 bytes
    // keeps both the 8-byte writes and the 16-byte reads free of bank
    // conflicts.  Rows past Sq are staged but not stored.
    constexpr int SROW = D * 2 + 16;
    static_assert(32 * SROW <= C::KTILE && 32 * SROW <= C::VTILE, "a wave's rows fit one tile buffer");
    char *stage = (wave_s == 0) ? k_lds0 : (wave_s == 1) ? k_lds1 : (wave_s == 2) ? v_lds0 : v_lds1;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                         pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        *(u32x2 *)(stage + l32 * SROW + (32 * db + 8 * g + 4 * h) * 2) = w;
      }
    }
    constexpr int CPR16 = D / 8;          // 16-byte chunks per row
    constexpr int RPS = 64 / CPR16;       // rows per store
    const int rr = lane / CPR16, cc = lane % CPR16;
#pragma unroll
    for (int i = 0; i < 32 / RPS; ++i) {
      const int row = RPS * i + rr;
      const u32x4 w = *(const u32x4 *)(stage + row * SROW + cc * 16);
      if (qw0 + row < a.Sq) *(u32x4 *)((__bf16 *)a.out + q_base + (size_t)(qw0 + row) * D + cc * 8) = w;
    }
  }
  if (qi < a.Sq) {
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
    }
    if (h == 0) {
      a.lse[(size_t)(b * a.Hq + hq) * a.Sq + qi] =
          (l_tot > 0.0f) ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int MASK, int MOD, bool OUT_F32>
hipError_t launch_variant(const KernelArgs &a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, MASK, MOD, OUT_F32>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, int MOD, bool OUT_F32>
hipError_t launch_mask(const KernelArgs &a, int mask, unsigned grid, hipStream_t stream) {
  switch (mask) {
    case ATTN_MASK_NONE: return launch_variant<D, ATTN_MASK_NONE, MOD, OUT_F32>(a, grid, stream);
    case ATTN_MASK_CAUSAL: return launch_variant<D, ATTN_MASK_CAUSAL, MOD, OUT_F32>(a, grid, stream);
    case ATTN_MASK_SLIDING: return launch_variant<D, ATTN_MASK_SLIDING, MOD, OUT_F32>(a, grid, stream);
    case ATTN_MASK_PREFIX_LM: return launch_variant<D, ATTN_MASK_PREFIX_LM, MOD, OUT_F32>(a, grid, stream);
    case ATTN_MASK_DOCUMENT: return launch_variant<D, ATTN_MASK_DOCUMENT, MOD, OUT_F32>(a, grid, stream);
    case kMaskDocWindow: return launch_variant<D, kMaskDocWindow, MOD, OUT_F32>(a, grid, stream);
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
  // Grouped heads in fours when the analytic key range applies (a BlockMask
  // row covers 128 query rows, so BlockMask launches keep the 128-row tile).
  a.gqa_pack = (p.bm_num == nullptr && p.Hkv > 0 && (p.Hq / p.Hkv) % 4 == 0) ? 1 : 0;
  const int rows = a.gqa_pack ? 32 : kBM;
  a.n_qtiles = (p.Sq + rows - 1) / rows;
  a.scale_log2 = p.scale * kLog2e;
  a.mask = p.mask;
  a.score = p.score;
  a.bm_num = p.bm_num;
  a.bm_idx = p.bm_idx;
  a.bm_full = p.bm_full;
  a.bm_nqb = p.bm_nqb;
  a.bm_nkb = p.bm_nkb;
  a.bm_batch = p.bm_batch;
  const unsigned grid = (unsigned)(a.n_qtiles * p.B * (a.gqa_pack ? p.Hq / 4 : p.Hq));
  if (p.score.kind == ATTN_SCORE_SOFTCAP) {
    return p.out_f32 ? launch_mask<D, kModCap, true>(a, p.mask.kind, grid, stream)
                     : launch_mask<D, kModCap, false>(a, p.mask.kind, grid, stream);
  }
  // The raw-score and linear-bias paths need a positive scale.
  if (!(a.scale_log2 > 0.0f)) {
    return p.out_f32 ? launch_mask<D, kModBias, true>(a, p.mask.kind, grid, stream)
                     : launch_mask<D, kModBias, false>(a, p.mask.kind, grid, stream);
  }
  if (p.score.kind != ATTN_SCORE_NONE) {   // ALIBI, REL_POS: a (j - i)
    return p.out_f32 ? launch_mask<D, kModLin, true>(a, p.mask.kind, grid, stream)
                     : launch_mask<D, kModLin, false>(a, p.mask.kind, grid, stream);
  }
  return p.out_f32 ? launch_mask<D, kModRaw, true>(a, p.mask.kind, grid, stream)
                   : launch_mask<D, kModRaw, false>(a, p.mask.kind, grid, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams &p, hipStream_t stream) {
  if (p.D == 64) return launch_d<64>(p, stream);
  if (p.D == 128) return launch_d<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
