// C ABI of the attention library: argument validation, kernel selection and
// launch on the caller's stream.  Every check runs on the host before any
// launch; the library allocates nothing and never synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool valid_mask_kind(int mk) { return mk >= ATTN_MASK_NONE && mk <= ATTN_MASK_AND; }

// The kind a set of intersected kinds (bit 1 << kind each) reduces to:
// SLIDING and DOCUMENT both imply j <= i, so CAUSAL adds nothing to either,
// and (j <= i or j < P) holds wherever j <= i does, so PREFIX_LM adds nothing
// to any of CAUSAL, SLIDING, DOCUMENT.  What is left is one kind, or SLIDING
// and DOCUMENT together.
int reduce_and(uint32_t bits) {
  const bool win = bits & (1u << ATTN_MASK_SLIDING);
  const bool doc = bits & (1u << ATTN_MASK_DOCUMENT);
  if (win && doc) return attn::kMaskDocWindow;
  if (doc) return ATTN_MASK_DOCUMENT;
  if (win) return ATTN_MASK_SLIDING;
  if (bits & (1u << ATTN_MASK_CAUSAL)) return ATTN_MASK_CAUSAL;
  if (bits & (1u << ATTN_MASK_PREFIX_LM)) return ATTN_MASK_PREFIX_LM;
  return ATTN_MASK_NONE;
}
bool valid_score_kind(int sk) { return sk >= ATTN_SCORE_NONE && sk <= ATTN_SCORE_SOFTCAP; }

// Shared checks of mask parameters; fills the kernel-side copy, with an AND
// set reduced to the kind the kernels run.  The parameters of every kind in
// the set are checked, also those the reduction drops.
int check_mask(int mk, const attn_mask_params_t *mp, int Sq, int Skv, attn::MaskArgs *out) {
  if (!valid_mask_kind(mk)) return fail(ATTN_ERR_INVALID, "unknown mask kind %d", mk);
  uint32_t bits = 1u << mk;
  if (mk == ATTN_MASK_AND) {
    if (!mp) return fail(ATTN_ERR_INVALID, "AND mask needs mask params");
    bits = mp->and_kinds;
    if (bits & ~0x1Fu) return fail(ATTN_ERR_INVALID, "and_kinds 0x%x names no mask kind", bits);
  }
  out->kind = reduce_and(bits);
  out->window = 0;
  out->prefix_len = 0;
  out->doc_ids = nullptr;
  out->doc_stride = Skv;
  if (bits & (1u << ATTN_MASK_SLIDING)) {
    if (!mp) return fail(ATTN_ERR_INVALID, "SLIDING mask needs mask params");
    if (mp->window < 1) return fail(ATTN_ERR_INVALID, "window must be >= 1 (got %d)", mp->window);
    out->window = mp->window;
  }
  if (bits & (1u << ATTN_MASK_PREFIX_LM)) {
    if (!mp) return fail(ATTN_ERR_INVALID, "PREFIX_LM mask needs mask params");
    if (mp->prefix_len < 0) return fail(ATTN_ERR_INVALID, "prefix_len must be >= 0");
    out->prefix_len = mp->prefix_len;
  }
  if (bits & (1u << ATTN_MASK_DOCUMENT)) {
    if (!mp || !mp->doc_ids) return fail(ATTN_ERR_INVALID, "DOCUMENT mask needs doc_ids");
    if (Sq != Skv) return fail(ATTN_ERR_UNSUPPORTED, "DOCUMENT mask needs Sq == Skv");
    out->doc_ids = mp->doc_ids;
  }
  return ATTN_OK;
}

int check_score(int sk, const attn_score_params_t *sp, attn::ScoreArgs *out) {
  if (!valid_score_kind(sk)) return fail(ATTN_ERR_INVALID, "unknown score kind %d", sk);
  out->kind = sk;
  out->slopes = sp ? sp->alibi_slopes : nullptr;
  out->rel_scale = sp ? sp->rel_scale : 1.0f;
  out->softcap = sp ? sp->softcap : 0.0f;
  if (sk == ATTN_SCORE_REL_POS && !sp) return fail(ATTN_ERR_INVALID, "REL_POS needs score params");
  if (sk == ATTN_SCORE_SOFTCAP) {
    if (!sp) return fail(ATTN_ERR_INVALID, "SOFTCAP needs score params");
    if (!(sp->softcap > 0.0f) || !std::isfinite(sp->softcap))
      return fail(ATTN_ERR_INVALID, "SOFTCAP needs a finite cap > 0 (got %g)", (double)sp->softcap);
  }
  return ATTN_OK;
}

int launch_result(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return ATTN_OK;
}

}  // namespace

namespace {

// Validation shared by the two decode entry points; fills everything of p
// but the workspace.  Returns ATTN_OK, an error, or 1 for an empty problem
// (nothing to launch).
int decode_prepare(const void *q, const void *k_cache, const void *v_cache, const int32_t *page_table,
                   const int32_t *seq_lens, void *out, float *lse, attn_dtype_t dt, int N, int Hq,
                   int Hkv, int D, int page_size, int max_pages_per_seq, int num_pages, float scale,
                   attn_mask_kind_t mk, const attn_mask_params_t *mp, attn_score_kind_t sk,
                   const attn_score_params_t *sp, attn::DecodeParams *p) {
  if (N < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || max_pages_per_seq <= 0 ||
      num_pages < 0)
    return fail(ATTN_ERR_INVALID, "bad size (N=%d Hq=%d Hkv=%d D=%d page=%d max_pages=%d pool=%d)",
                N, Hq, Hkv, D, page_size, max_pages_per_seq, num_pages);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (dt != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "paged decode supports bf16 only");
  if (D != 128) return fail(ATTN_ERR_UNSUPPORTED, "paged decode supports D == 128 (got %d)", D);
  if (page_size != 16) return fail(ATTN_ERR_UNSUPPORTED, "paged decode supports page_size == 16");
  if (Hq / Hkv > 16) return fail(ATTN_ERR_UNSUPPORTED, "paged decode supports Hq/Hkv <= 16");
  int rc = check_mask(mk, mp, 1, 1, &p->mask);
  if (rc) return rc;
  if (p->mask.kind != ATTN_MASK_NONE && p->mask.kind != ATTN_MASK_SLIDING)
    return fail(ATTN_ERR_UNSUPPORTED, "paged decode supports no mask or a sliding window");
  rc = check_score(sk, sp, &p->score);
  if (rc) return rc;
  if (N == 0) {
    g_err[0] = '\0';
    return 1;
  }
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !out || !lse)
    return fail(ATTN_ERR_INVALID, "null tensor pointer");
  p->q = q;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  p->page_table = page_table;
  p->seq_lens = seq_lens;
  p->out = out;
  p->lse = lse;
  p->N = N;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->D = D;
  p->page_size = page_size;
  p->max_pages = max_pages_per_seq;
  p->num_pages = num_pages;
  p->scale = scale;
  return ATTN_OK;
}

// Bytes of split partials for `splits` splits per (sequence, query head):
// fp32 rows of D, rounded up to 256 bytes, then one fp32 LSE per row.
size_t decode_partials_bytes(int N, int Hq, int D, int splits) {
  const size_t rows = (size_t)N * Hq * splits;
  return (rows * D * sizeof(float) + 255) / 256 * 256 + rows * sizeof(float);
}

void decode_set_workspace(attn::DecodeParams *p, void *base, int splits) {
  const size_t rows = (size_t)p->N * p->Hq * splits;
  p->ws_o = (float *)base;
  p->ws_lse = (float *)((char *)base + (rows * p->D * sizeof(float) + 255) / 256 * 256);
  p->max_splits = splits;
}

// Scratch of attn_paged_decode_noalloc, for callers that cannot allocate:
// one array per GPU, held for the life of the process.  Host code never
// takes the array's own address (on the host it is only a stand-in for the
// symbol); it uses the device address hipGetSymbolAddress returns, looked up
// once per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (the device the stream belongs to,
// which must be the current one).
int scratch_address(hipStream_t stream, void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(ATTN_ERR_INVALID, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(ATTN_ERR_INVALID, "the stream belongs to device %d but device %d is current", (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !addr)
      return fail(ATTN_ERR_LAUNCH, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = addr;
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char *attn_last_error(void) { return g_err; }

int attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
             attn_dtype_t dt, attn_dtype_t out_dt, int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
             attn_mask_kind_t mk, const attn_mask_params_t *mp, attn_score_kind_t sk,
             const attn_score_params_t *sp, const attn_block_mask_t *bm, void *stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || D <= 0)
    return fail(ATTN_ERR_INVALID, "negative size (B=%d Hq=%d Hkv=%d Sq=%d Skv=%d D=%d)", B, Hq,
                Hkv, Sq, Skv, D);
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0))
    return fail(ATTN_ERR_INVALID, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  if (dt != ATTN_BF16 && dt != ATTN_F32) return fail(ATTN_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (out_dt != ATTN_BF16 && out_dt != ATTN_F32)
    return fail(ATTN_ERR_INVALID, "unknown output dtype %d", (int)out_dt);
  if (dt == ATTN_F32 && out_dt != ATTN_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "fp32 inputs need an fp32 output");
  if (dt == ATTN_BF16 && D != 64 && D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "bf16 path supports D in {64, 128} (got %d)", D);
  if (dt == ATTN_BF16 && (int64_t)Skv * D * 2 > 2147483647LL)
    return fail(ATTN_ERR_UNSUPPORTED, "bf16 path needs Skv * D * 2 < 2^31 bytes per head");
  if (dt == ATTN_F32 && D != 16 && D != 32 && D != 64 && D != 128 && D != 256)
    return fail(ATTN_ERR_UNSUPPORTED, "fp32 path supports D in {16, 32, 64, 128, 256} (got %d)", D);
  attn::FwdParams p{};
  int rc = check_mask(mk, mp, Sq, Skv, &p.mask);
  if (rc) return rc;
  rc = check_score(sk, sp, &p.score);
  if (rc) return rc;
  if (!(scale == scale)) return fail(ATTN_ERR_INVALID, "scale is NaN");
  if (bm) {
    if (!bm->kv_num_blocks || !bm->kv_indices)
      return fail(ATTN_ERR_INVALID, "block mask needs kv_num_blocks and kv_indices");
    if (bm->q_block != 128 || bm->kv_block != 128)
      return fail(ATTN_ERR_UNSUPPORTED, "block mask must use 128 x 128 blocks (got %d x %d)",
                  bm->q_block, bm->kv_block);
    if (bm->n_q_blocks != (Sq + 127) / 128 || bm->n_kv_blocks != (Skv + 127) / 128)
      return fail(ATTN_ERR_INVALID, "block mask shape %d x %d does not match Sq=%d Skv=%d",
                  bm->n_q_blocks, bm->n_kv_blocks, Sq, Skv);
    if (dt == ATTN_BF16 && bm->n_kv_blocks > 1024)
      return fail(ATTN_ERR_UNSUPPORTED, "block mask with more than 1024 key blocks (Skv > 131072)");
    if (bm->batch != 1 && bm->batch != B)
      return fail(ATTN_ERR_INVALID, "block mask batch %d must be 1 or B=%d", bm->batch, B);
    p.bm_num = bm->kv_num_blocks;
    p.bm_idx = bm->kv_indices;
    p.bm_full = bm->kv_full;
    p.bm_nqb = bm->n_q_blocks;
    p.bm_nkb = bm->n_kv_blocks;
    p.bm_batch = bm->batch;
    p.bm_kv_block = bm->kv_block;
  }
  if (B == 0 || Hq == 0 || Sq == 0) {
    g_err[0] = '\0';
    return ATTN_OK;
  }
  if (!q || !out || !lse || (Skv > 0 && (!k || !v)))
    return fail(ATTN_ERR_INVALID, "null tensor pointer");
  const double rows = (double)B * Hq * ((Sq + 127) / 128);
  if (rows > 2147483647.0) return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Skv = Skv;
  p.D = D;
  p.out_f32 = (out_dt == ATTN_F32);
  p.scale = scale;
  hipStream_t s = (hipStream_t)stream;
  if (dt == ATTN_BF16) return launch_result(attn::launch_fwd_bf16(p, s), "attn_fwd (bf16)");
  return launch_result(attn::launch_fwd_f32(p, s), "attn_fwd (fp32)");
}

int attn_build_block_mask(attn_mask_kind_t mk, const attn_mask_params_t *mp, int B, int Sq,
                          int Skv, int q_block, int kv_block, int32_t *kv_num_blocks,
                          int32_t *kv_indices, uint8_t *kv_full, void *stream) {
  if (B < 0 || Sq < 0 || Skv < 0) return fail(ATTN_ERR_INVALID, "negative size");
  if (q_block < 16 || q_block > 1024 || q_block % 16 || kv_block < 16 || kv_block > 1024 ||
      kv_block % 16)
    return fail(ATTN_ERR_UNSUPPORTED, "block sizes must be multiples of 16 in [16, 1024]");
  attn::BlockMaskParams p{};
  int rc = check_mask(mk, mp, Sq, Skv, &p.mask);
  if (rc) return rc;
  if (B == 0 || Sq == 0) {
    g_err[0] = '\0';
    return ATTN_OK;
  }
  if (!kv_num_blocks || (Skv > 0 && !kv_indices)) return fail(ATTN_ERR_INVALID, "null output pointer");
  p.B = B;
  p.Sq = Sq;
  p.Skv = Skv;
  p.q_block = q_block;
  p.kv_block = kv_block;
  p.nqb = (Sq + q_block - 1) / q_block;
  p.nkb = (Skv + kv_block - 1) / kv_block;
  p.num = kv_num_blocks;
  p.idx = kv_indices;
  p.full = kv_full;
  return launch_result(attn::launch_block_mask(p, (hipStream_t)stream), "attn_build_block_mask");
}

size_t attn_paged_decode_workspace_size(int num_seqs, int Hq, int D, int max_pages_per_seq,
                                        int page_size) {
  (void)page_size;
  if (num_seqs <= 0 || Hq <= 0 || D <= 0 || max_pages_per_seq <= 0) return 0;
  const size_t rows = (size_t)num_seqs * Hq * attn::decode_max_splits(max_pages_per_seq);
  const size_t o_bytes = (rows * D * sizeof(float) + 255) / 256 * 256;
  return o_bytes + rows * sizeof(float);
}

int attn_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *page_table, const int32_t *seq_lens, void *out, float *lse,
                      attn_dtype_t dt, int N, int Hq, int Hkv, int D, int page_size,
                      int max_pages_per_seq, int num_pages, float scale, attn_mask_kind_t mk,
                      const attn_mask_params_t *mp, attn_score_kind_t sk,
                      const attn_score_params_t *sp, void *workspace, size_t workspace_bytes,
                      void *stream) {
  attn::DecodeParams p{};
  int rc = decode_prepare(q, k_cache, v_cache, page_table, seq_lens, out, lse, dt, N, Hq, Hkv, D,
                          page_size, max_pages_per_seq, num_pages, scale, mk, mp, sk, sp, &p);
  if (rc) return rc == 1 ? ATTN_OK : rc;
  const size_t need = attn_paged_decode_workspace_size(N, Hq, D, max_pages_per_seq, page_size);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace) % 256 != 0) return fail(ATTN_ERR_INVALID, "workspace must be 256-byte aligned");
  decode_set_workspace(&p, workspace, attn::decode_max_splits(max_pages_per_seq));
  return launch_result(attn::launch_paged_decode(p, (hipStream_t)stream), "attn_paged_decode");
}

int attn_paged_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *page_table, const int32_t *seq_lens, void *out, float *lse,
                              attn_dtype_t dt, int N, int Hq, int Hkv, int D, int page_size,
                              int max_pages_per_seq, int num_pages, float scale, attn_mask_kind_t mk,
                              const attn_mask_params_t *mp, attn_score_kind_t sk,
                              const attn_score_params_t *sp, void *stream) {
  attn::DecodeParams p{};
  int rc = decode_prepare(q, k_cache, v_cache, page_table, seq_lens, out, lse, dt, N, Hq, Hkv, D,
                          page_size, max_pages_per_seq, num_pages, scale, mk, mp, sk, sp, &p);
  if (rc) return rc == 1 ? ATTN_OK : rc;
  // Only the splits this launch takes need room (the workspace of
  // attn_paged_decode is sized for the smallest split size instead).
  const int splits = attn::decode_launch_splits(p);
  const size_t need = decode_partials_bytes(N, Hq, D, splits);
  if (need > kScratchBytes)
    return fail(ATTN_ERR_WORKSPACE,
                "attn_paged_decode_noalloc: %d sequences x %d heads x %d splits need %zu bytes of "
                "scratch, more than its fixed %zu",
                N, Hq, splits, need, kScratchBytes);
  void *base = nullptr;
  rc = scratch_address((hipStream_t)stream, &base);
  if (rc) return rc;
  decode_set_workspace(&p, base, splits);
  return launch_result(attn::launch_paged_decode(p, (hipStream_t)stream), "attn_paged_decode_noalloc");
}

int attn_block_mask_transpose(const attn_block_mask_t *bm, int32_t *q_num_blocks, int32_t *q_indices,
                              uint8_t *q_full, void *stream) {
  if (!bm) return fail(ATTN_ERR_INVALID, "null block mask");
  if (bm->batch < 0 || bm->n_q_blocks < 0 || bm->n_kv_blocks < 0)
    return fail(ATTN_ERR_INVALID, "negative block mask shape");
  if (bm->batch == 0 || bm->n_kv_blocks == 0) {
    g_err[0] = '\0';
    return ATTN_OK;
  }
  if (!q_num_blocks || (bm->n_q_blocks > 0 && !q_indices)) return fail(ATTN_ERR_INVALID, "null output pointer");
  if (bm->n_q_blocks > 0 && (!bm->kv_num_blocks || !bm->kv_indices))
    return fail(ATTN_ERR_INVALID, "block mask needs kv_num_blocks and kv_indices");
  attn::BlockMaskTransposeParams p{};
  p.num = bm->kv_num_blocks;
  p.idx = bm->kv_indices;
  p.full = bm->kv_full;
  p.q_num = q_num_blocks;
  p.q_idx = q_indices;
  p.q_full = q_full;
  p.batch = bm->batch;
  p.nqb = bm->n_q_blocks;
  p.nkb = bm->n_kv_blocks;
  return launch_result(attn::launch_block_mask_transpose(p, (hipStream_t)stream), "attn_block_mask_transpose");
}

size_t attn_bwd_workspace_size(int B, int Hq, int Sq) {
  if (B <= 0 || Hq <= 0 || Sq <= 0) return 0;
  return ((size_t)B * Hq * Sq * sizeof(float) + 255) / 256 * 256;
}

int attn_bwd(const void *q, const void *k, const void *v, const void *out, const float *lse,
             const void *dout, float *dq, float *dk, float *dv, attn_dtype_t dt, int B, int Hq, int Hkv,
             int Sq, int Skv, int D, float scale, attn_mask_kind_t mk, const attn_mask_params_t *mp,
             attn_score_kind_t sk, const attn_score_params_t *sp, const attn_block_mask_t *bm,
             void *workspace, size_t workspace_bytes, void *stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || D <= 0)
    return fail(ATTN_ERR_INVALID, "negative size (B=%d Hq=%d Hkv=%d Sq=%d Skv=%d D=%d)", B, Hq,
                Hkv, Sq, Skv, D);
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0))
    return fail(ATTN_ERR_INVALID, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  if (dt != ATTN_BF16 && dt != ATTN_F32) return fail(ATTN_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (dt != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "the backward supports bf16 inputs only");
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "the backward supports D in {64, 128} (got %d)", D);
  if ((int64_t)Skv * D * 2 > 2147483647LL || (int64_t)Sq * D * 2 > 2147483647LL)
    return fail(ATTN_ERR_UNSUPPORTED, "the backward needs Sq, Skv * D * 2 < 2^31 bytes per head");
  attn::BwdParams p{};
  int rc = check_mask(mk, mp, Sq, Skv, &p.mask);
  if (rc) return rc;
  rc = check_score(sk, sp, &p.score);
  if (rc) return rc;
  if (!(scale == scale)) return fail(ATTN_ERR_INVALID, "scale is NaN");
  if (bm) {
    if (!bm->kv_num_blocks || !bm->kv_indices || !bm->q_num_blocks || !bm->q_indices)
      return fail(ATTN_ERR_INVALID, "the backward needs the block mask lists both ways "
                                    "(attn_block_mask_transpose writes the ones by key block)");
    if (bm->q_block != 128 || bm->kv_block != 128)
      return fail(ATTN_ERR_UNSUPPORTED, "block mask must use 128 x 128 blocks (got %d x %d)",
                  bm->q_block, bm->kv_block);
    if (bm->n_q_blocks != (Sq + 127) / 128 || bm->n_kv_blocks != (Skv + 127) / 128)
      return fail(ATTN_ERR_INVALID, "block mask shape %d x %d does not match Sq=%d Skv=%d",
                  bm->n_q_blocks, bm->n_kv_blocks, Sq, Skv);
    if (bm->n_kv_blocks > 1024 || bm->n_q_blocks > 1024)
      return fail(ATTN_ERR_UNSUPPORTED, "block mask with more than 1024 blocks a side");
    if (bm->batch != 1 && bm->batch != B)
      return fail(ATTN_ERR_INVALID, "block mask batch %d must be 1 or B=%d", bm->batch, B);
    p.bm_num = bm->kv_num_blocks;
    p.bm_idx = bm->kv_indices;
    p.bm_full = bm->kv_full;
    p.bm_qnum = bm->q_num_blocks;
    p.bm_qidx = bm->q_indices;
    p.bm_qfull = bm->q_full;
    p.bm_nqb = bm->n_q_blocks;
    p.bm_nkb = bm->n_kv_blocks;
    p.bm_batch = bm->batch;
  }
  if (B == 0 || Hq == 0 || (Sq == 0 && Skv == 0)) {
    g_err[0] = '\0';
    return ATTN_OK;
  }
  const size_t need = attn_bwd_workspace_size(B, Hq, Sq);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace) % 256 != 0) return fail(ATTN_ERR_INVALID, "workspace must be 256-byte aligned");
  if ((Sq > 0 && (!q || !out || !lse || !dout || !dq)) || (Skv > 0 && (!k || !v || !dk || !dv)))
    return fail(ATTN_ERR_INVALID, "null tensor pointer");
  const double grid = (double)B * Hq * ((Sq + 127) / 128) + (double)B * Hkv * ((Skv + 127) / 128);
  if (grid > 2147483647.0) return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.row_dot = (float *)workspace;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Skv = Skv;
  p.D = D;
  p.scale = scale;
  return launch_result(attn::launch_bwd_bf16(p, (hipStream_t)stream), "attn_bwd");
}

}  // extern "C"
