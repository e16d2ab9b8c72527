/*
 * attn_fa2.h — C ABI of the MI355X (gfx950) fused-attention library.
 *
 * The operation is softmax attention with a per-score modifier applied before
 * the softmax and a visibility mask, as stated in the FlexAttention write-up
 * "新PyTorch API：几行代码实现不同注意力变体，兼具FlashAttention性能和PyTorch
 * 灵活性" (§FlexAttention: softmax(score_mod(Q·Kᵀ))·V with
 * score_mod(score, b, h, q_idx, kv_idx)), computed in one pass with an
 * online softmax (the 1-pass FlashAttention form of "Attention优化｜2w字原理
 * &图解: 从Online-Softmax到FlashAttention V1/V2/V3", abstract), plus a
 * block-sparse mask that lets the kernel skip masked key tiles (same
 * write-up, introduction: exploiting mask sparsity) and a paged-KV decode
 * (PagedAttention in the write-up's variant list).
 *
 * Conventions common to every call:
 *  - Every tensor pointer is caller-owned DEVICE memory, contiguous,
 *    row-major, in the layout stated per argument.  The library never
 *    allocates, frees or keeps a pointer after it returns, and never
 *    synchronises: work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream) and the caller keeps the buffers alive until the stream
 *    has reached it.  The one piece of device memory it owns is the fixed
 *    per-GPU scratch of attn_paged_decode_noalloc, part of the loaded code
 *    object.
 *  - Return value: 0 on success, negative on failure:
 *      ATTN_ERR_INVALID     (-1) a null pointer, a negative or inconsistent size;
 *      ATTN_ERR_UNSUPPORTED (-2) a valid request outside the supported set;
 *      ATTN_ERR_LAUNCH      (-3) the HIP runtime rejected a launch;
 *      ATTN_ERR_WORKSPACE   (-4) the workspace is too small.
 *    All argument checks run on the host before any launch, so nothing is
 *    written on error.  A device fault surfaces at the caller's next
 *    synchronisation (HIP semantics).  attn_last_error() returns a message
 *    for the last failed call on the calling thread.
 *  - Indices are raw row / column numbers (the page's score_mod loop runs
 *    q_idx and kv_idx over positions from 0).
 */
#ifndef ATTN_FA2_H
#define ATTN_FA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_ERR_INVALID (-1)
#define ATTN_ERR_UNSUPPORTED (-2)
#define ATTN_ERR_LAUNCH (-3)
#define ATTN_ERR_WORKSPACE (-4)

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Mask predicates (FlexAttention write-up: §Causal Mask, §Sliding Window +
 * Causal, and the PrefixLM / document-mask entries of its variant list).
 * visible(b, i, j) for query i, key j:
 *   NONE      always
 *   CAUSAL    j <= i
 *   SLIDING   0 <= i - j < window            (causal + window of `window` keys, self included)
 *   PREFIX_LM j <= i  or  j < prefix_len
 *   DOCUMENT  doc_ids[b, i] == doc_ids[b, j]  and  j <= i
 *   AND       every kind k with bit (1u << k) set in and_kinds holds, each with
 *             the same params (the variant list's combination "sliding
 *             window + document + causal" is and_kinds = SLIDING | DOCUMENT |
 *             CAUSAL bits); no bit set means no mask.  Bits other than those
 *             of NONE..DOCUMENT are an error.  The set is reduced exactly
 *             before launch: CAUSAL adds nothing to SLIDING or DOCUMENT (both
 *             imply j <= i), PREFIX_LM adds nothing to a kind that implies
 *             j <= i, so every set is one of the kinds above or SLIDING and
 *             DOCUMENT together.                                              */
typedef enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_SLIDING = 2,
  ATTN_MASK_PREFIX_LM = 3,
  ATTN_MASK_DOCUMENT = 4,
  ATTN_MASK_AND = 5
} attn_mask_kind_t;

typedef struct {
  int32_t window;          /* SLIDING: number of keys, >= 1 */
  int32_t prefix_len;      /* PREFIX_LM: bidirectional prefix length, >= 0 */
  const int32_t *doc_ids;  /* DOCUMENT: device int32 [B, S] (Sq == Skv == S) */
  uint32_t and_kinds;      /* AND: bit (1u << kind) per intersected kind */
} attn_mask_params_t;

/* Score modifiers, applied to the scaled score x = scale * q.k before the
 * mask and softmax (FlexAttention write-up §FlexAttention: score_mod on every
 * score; §相对位置编码: a bias from the query-key distance computed inside
 * the kernel, never stored as an S x S tensor; ALiBi from the variant list;
 * §Soft-capping, formula lost, read as below):
 *   NONE     x
 *   ALIBI    x + slope[hq] * (j - i),  slope[h] = 2^(-8 (h+1) / Hq) by default
 *   REL_POS  x + rel_scale * (i - j)
 *   SOFTCAP  softcap * tanh(x / softcap), softcap > 0 and finite            */
typedef enum {
  ATTN_SCORE_NONE = 0,
  ATTN_SCORE_ALIBI = 1,
  ATTN_SCORE_REL_POS = 2,
  ATTN_SCORE_SOFTCAP = 3
} attn_score_kind_t;

typedef struct {
  const float *alibi_slopes; /* device float [Hq], or NULL for 2^(-8(h+1)/Hq) */
  float rel_scale;           /* REL_POS constant c */
  float softcap;             /* SOFTCAP cap (> 0, finite) */
} attn_score_params_t;

/* Block-sparse mask over q_block x kv_block blocks of the Sq x Skv grid (the
 * last blocks clipped at Sq / Skv).  For batch b (0 when batch == 1, which
 * broadcasts) and query block qb:
 *   kv_num_blocks[b, 0, qb]      number of listed key blocks
 *   kv_indices[b, 0, qb, n]      listed key blocks, ascending; -1 past the count
 *   kv_full[b, 0, qb, n]         1 if every (i, j) of that block is visible
 *                                (the kernel then skips the predicate); may be NULL
 * All device memory; shapes [batch, 1, n_q_blocks(, n_kv_blocks)].          */
typedef struct {
  const int32_t *kv_num_blocks;
  const int32_t *kv_indices;
  const uint8_t *kv_full;
  int32_t q_block, kv_block, n_q_blocks, n_kv_blocks, batch;
  /* The same incidence by key block, for attn_bwd's key-stationary pass
   * (attn_block_mask_transpose writes them; attn_fwd ignores them):
   *   q_num_blocks[b, 0, kb]   number of query blocks that list kb
   *   q_indices[b, 0, kb, n]   those query blocks, ascending; -1 past the count
   *   q_full[b, 0, kb, n]      their full flags; may be NULL                 */
  const int32_t *q_num_blocks;
  const int32_t *q_indices;
  const uint8_t *q_full;
} attn_block_mask_t;

/* attn_fwd — fused attention forward, one pass with online softmax.
 *
 *   q   [B, Hq,  Sq,  D]   dtype `dt`
 *   k   [B, Hkv, Skv, D]   dtype `dt`
 *   v   [B, Hkv, Skv, D]   dtype `dt`
 *   out [B, Hq,  Sq,  D]   dtype `out_dt` (written): the input dtype, or
 *                          F32 for bf16 inputs (the fp32 value before the
 *                          final rounding; a bf16 `out` is exactly that value
 *                          rounded to nearest even)
 *   lse [B, Hq,  Sq]       float32, natural-log log-sum-exp of each row's
 *                          modified scores (written; -inf for a row with no
 *                          visible key, whose output row is 0)
 *   Query head hq reads kv head floor(hq * Hkv / Hq) (Hq % Hkv == 0).
 *   S[i,j] = scale * q_i·k_j + bias(hq, i, j), masked to -inf where not
 *   visible; out_i = softmax(S[i,:]) · V; lse_i = ln sum_j e^{S[i,j]}.
 *   bm: NULL iterates the key tiles the mask kind allows analytically;
 *   otherwise only the listed blocks are visited and the mask predicate is
 *   evaluated on blocks not flagged full (the caller keeps bm consistent with
 *   mk: a block left out is treated as fully masked).
 * Supported: dt = BF16 with D in {64, 128} (MFMA path, fp32 accumulation,
 * P rounded to bf16 before P·V) or dt = F32 with D in {16, 32, 64, 128, 256}
 * (fp32 path); bm with q_block == kv_block == 128 (and, on the bf16 path,
 * at most 1024 key blocks, Skv <= 131072); DOCUMENT needs
 * Sq == Skv.  Returns 0 for B, Sq or Hq equal to 0 without launching.     */
int attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
             attn_dtype_t dt, attn_dtype_t out_dt, int B, int Hq, int Hkv, int Sq, int Skv, int D,
             float scale, attn_mask_kind_t mk, const attn_mask_params_t *mp,
             attn_score_kind_t sk, const attn_score_params_t *sp,
             const attn_block_mask_t *bm, void *stream);

/* attn_build_block_mask — BlockMask of mask kind `mk` (same predicate as
 * attn_fwd) for B x Sq x Skv, in q_block x kv_block blocks.  The FlexAttention
 * write-up's introduction says the kernel exploits the sparsity of the mask
 * by skipping fully masked blocks; this call computes that block structure
 * once, for reuse by every attn_fwd / attn_bwd call with the same mask (the
 * write-up gives no layout: the one below, per query block an ascending list
 * of the key blocks that hold a visible pair plus a flag for blocks where
 * every pair is visible, is this library's).
 *   kv_num_blocks int32 [B, 1, ceil(Sq/q_block)]                 (written)
 *   kv_indices    int32 [B, 1, ceil(Sq/q_block), ceil(Skv/kv_block)] (written)
 *   kv_full       uint8 same shape as kv_indices, or NULL         (written)
 * Listed: a block holding at least one visible (i, j); full: all visible.
 * Lists ascend; unused tails are -1 (indices) and 0 (full).  Bit-exact.
 * Supported: q_block, kv_block in [16, 1024], multiples of 16.             */
int attn_build_block_mask(attn_mask_kind_t mk, const attn_mask_params_t *mp, int B, int Sq,
                          int Skv, int q_block, int kv_block, int32_t *kv_num_blocks,
                          int32_t *kv_indices, uint8_t *kv_full, void *stream);

/* attn_block_mask_transpose — the lists of bm by key block (bm->q_*):
 * per key block kb, the ascending query blocks whose kv_indices hold kb and
 * their kv_full flags.  The backward's key-stationary pass walks these.
 * Reads bm->kv_num_blocks / kv_indices (ascending, as attn_build_block_mask
 * writes them) / kv_full (may be NULL: all flags 0); writes
 *   q_num_blocks int32 [batch, 1, n_kv_blocks]
 *   q_indices    int32 [batch, 1, n_kv_blocks, n_q_blocks], -1 tails
 *   q_full       uint8 [batch, 1, n_kv_blocks, n_q_blocks], 0 tails; may be NULL
 * device memory, caller-owned.  Errors: -1 for null pointers or a negative
 * shape.                                                                    */
int attn_block_mask_transpose(const attn_block_mask_t *bm, int32_t *q_num_blocks, int32_t *q_indices,
                              uint8_t *q_full, void *stream);

/* attn_bwd_workspace_size — bytes of device scratch attn_bwd needs (the
 * pages say nothing of it; this library's choice): one float per query row,
 * the row term D = rowsum(dO * O), B * Hq * Sq * 4, rounded up to 256.     */
size_t attn_bwd_workspace_size(int B, int Hq, int Sq);

/* attn_bwd — gradients of attn_fwd from its stored LSE.  The FlexAttention
 * write-up obtains its backward by automatic differentiation of the forward
 * (introduction) and runs a deterministic algorithm that recomputes more
 * than FlashAttention-2 (§性能); this one writes every gradient element from
 * one workgroup, without atomics, and recomputes P = exp(S - LSE).
 * With x = scale * q.k, S = score_mod(x) masked and P = softmax(S):
 *   dV = P^T dO,  dS = P (dO V^T - rowsum(dO * O)),
 *   dQ = scale * (dS score_mod'(x)) K,  dK = scale * (dS score_mod'(x))^T Q,
 * and a kv head's dK, dV sum every query head of its group.
 *   q, out, dout [B, Hq, Sq, D]; k, v [B, Hkv, Skv, D]       bf16, device
 *   lse          [B, Hq, Sq] float32: the forward's LSE (natural log)
 *   dq           [B, Hq, Sq, D]   float32 (written)
 *   dk, dv       [B, Hkv, Skv, D] float32 (written; zeros for keys no query sees)
 *   scale, mk/mp, sk/sp: those of the forward call (same meaning and checks)
 *   workspace: device scratch of at least attn_bwd_workspace_size(B, Hq, Sq)
 *   bytes, 256-byte aligned; caller-owned, contents on entry do not matter.
 * A row with no visible key contributes nothing.  Supported: dt = BF16,
 * D in {64, 128} (others return -2).
 *   bm: NULL, or the forward's BlockMask (128 x 128 blocks) with its lists
 *   by key block filled in (attn_block_mask_transpose): the dQ pass walks
 *   kv_indices, the dK/dV pass q_indices, and full flags drop the
 *   predicate.  It must describe the mask mk / mp (it only selects blocks).
 *   Without it, tiles are chosen from each mask's closed-form bounds and
 *   document ids are compared per element over the causal range.
 * Errors as attn_fwd, plus -4 for a short workspace.                        */
int attn_bwd(const void *q, const void *k, const void *v, const void *out, const float *lse,
             const void *dout, float *dq, float *dk, float *dv, attn_dtype_t dt, int B, int Hq, int Hkv,
             int Sq, int Skv, int D, float scale, attn_mask_kind_t mk, const attn_mask_params_t *mp,
             attn_score_kind_t sk, const attn_score_params_t *sp, const attn_block_mask_t *bm,
             void *workspace, size_t workspace_bytes, void *stream);

/* attn_paged_decode_workspace_size — bytes of device scratch attn_paged_decode
 * needs for this shape (the pages say nothing of a split-KV workspace; its
 * size and layout are this library's): fp32 partial outputs and
 * log-sum-exps of every key split, for splits as small as 16 pages (the launch takes 64-page splits,
 * or 32 / 16 when that leaves too few work items), sized from
 * max_pages_per_seq so the host never reads seq_lens:
 * N * Hq * ceil(max_pages_per_seq / 16) * (D + 1) * 4 bytes, plus padding. */
size_t attn_paged_decode_workspace_size(int num_seqs, int Hq, int D, int max_pages_per_seq,
                                        int page_size);

/* attn_paged_decode — one query per sequence against its paged KV cache
 * (PagedAttention, FlexAttention write-up variant list; the multi-query
 * paged-attention kernel of "高级特性：探索PyTorch/XLA的Pallas内核和Flash
 * Attention实现"), split over keys, then merged by log-sum-exp.
 *   q          [N, Hq, D]                     bf16
 *   k_cache    [num_pages, Hkv, page_size, D] bf16
 *   v_cache    [num_pages, Hkv, page_size, D] bf16
 *   num_pages  pages in the pool; a page id outside [0, num_pages) is read
 *              as a page of zeros instead of faulting
 *   page_table int32 [N, max_pages_per_seq]; token t of sequence s sits in
 *              page page_table[s, t / page_size], slot t % page_size;
 *              entries past ceil(seq_lens[s] / page_size) are never read
 *   seq_lens   int32 [N], each in [0, max_pages_per_seq * page_size]; a
 *              sequence of length 0 gets O = 0 and LSE = -inf
 *   out        [N, Hq, D] bf16 (written); lse [N, Hq] float32 (written)
 *   The query of sequence s sits at position i = seq_lens[s] - 1.  With
 *   mk = ATTN_MASK_NONE it sees every key t <= i; with ATTN_MASK_SLIDING
 *   (PagedAttention + sliding window, both in the FlexAttention write-up's
 *   variant list; window as in its §Sliding Window + Causal) it sees the
 *   keys with 0 <= i - t < mp->window: pages wholly before the window are
 *   never read, and what the slots of earlier keys hold (NaN included) has
 *   no effect.  ALIBI / REL_POS use i = seq_lens[s] - 1.
 *   workspace: device scratch of at least
 *   attn_paged_decode_workspace_size(...) bytes, 256-byte aligned.  When
 *   every key range fits 128 pages (max_pages_per_seq, or the window, small
 *   enough) and N * Hkv >= 256, each sequence is one work item written
 *   straight to out / lse and the workspace is not touched.
 * Supported: dt = BF16, D == 128, page_size == 16, Hq % Hkv == 0,
 * Hq / Hkv <= 16, mk in {NONE, SLIDING} (others return -2).               */
int attn_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *page_table, const int32_t *seq_lens, void *out, float *lse,
                      attn_dtype_t dt, int N, int Hq, int Hkv, int D, int page_size,
                      int max_pages_per_seq, int num_pages, float scale, attn_mask_kind_t mk,
                      const attn_mask_params_t *mp, attn_score_kind_t sk,
                      const attn_score_params_t *sp, void *workspace, size_t workspace_bytes,
                      void *stream);

/* attn_paged_decode_noalloc — attn_paged_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments, meaning,
 * checks, kernels and results, minus the workspace.  The split partials go
 * to a scratch array the library holds on each GPU for the life of the
 * process (64 MiB = 67,108,864 bytes); the first
 * call on a device looks its address up, with the stream's device current.
 * The call itself allocates nothing.
 *   Scratch needed: N * Hq * splits * (D + 1) * 4 bytes (plus padding),
 *   with splits = the key splits per sequence this launch takes (64 pages
 *   each, or 32 / 16 when that leaves too few work items), bounded by
 *   max_pages_per_seq and the window; 0 when each sequence is one work item
 *   written straight to the output (as attn_paged_decode).  A request needing more returns -4
 *   (ATTN_ERR_WORKSPACE) with the sizes in attn_last_error(); the 64-sequence,
 *   32-head, 2048-page shape needs 33.8 MB.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap
 *   on one GPU (different streams, or different host threads without
 *   ordering) race and may return wrong results; serialise them.  Nothing
 *   in the scratch has to start at zero (each call writes every partial it
 *   reads).  The stream must belong to the current device (else -1).        */
int attn_paged_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *page_table, const int32_t *seq_lens, void *out,
                              float *lse, attn_dtype_t dt, int N, int Hq, int Hkv, int D,
                              int page_size, int max_pages_per_seq, int num_pages, float scale,
                              attn_mask_kind_t mk, const attn_mask_params_t *mp,
                              attn_score_kind_t sk, const attn_score_params_t *sp, void *stream);

/* Message of the last failed call on this thread ("" if none); valid until
 * the next call on the thread. */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FA2_H */
