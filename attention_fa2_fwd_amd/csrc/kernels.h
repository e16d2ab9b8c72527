// Launch interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include "common.h"

namespace attn {

// Everything the forward kernels read, validated by the host first.
struct FwdParams {
  const void *q, *k, *v;
  void *out;
  float *lse;
  int B, Hq, Hkv, Sq, Skv, D;
  bool out_f32;   // bf16 path: write O as fp32 instead of bf16
  float scale;
  MaskArgs mask;
  ScoreArgs score;
  // BlockMask (bm_num == nullptr: analytic tile ranges)
  const int32_t *bm_num;
  const int32_t *bm_idx;
  const uint8_t *bm_full;
  int bm_nqb, bm_nkb, bm_batch, bm_kv_block;
};

// bf16 MFMA path, D in {64, 128}.
hipError_t launch_fwd_bf16(const FwdParams &p, hipStream_t stream);

struct BwdParams {
  const void *q, *k, *v, *out, *dout;   // bf16
  const float *lse;
  float *dq, *dk, *dv;
  float *row_dot;   // workspace [B, Hq, Sq]: sum_d dO * O, formed by the dQ kernel
  int B, Hq, Hkv, Sq, Skv, D;
  float scale;
  MaskArgs mask;
  ScoreArgs score;
  // BlockMask, 128 x 128 blocks (bm_num == nullptr: closed-form tile ranges):
  // lists by query block for the dQ pass, by key block for the dK/dV pass.
  const int32_t *bm_num, *bm_idx, *bm_qnum, *bm_qidx;
  const uint8_t *bm_full, *bm_qfull;
  int bm_nqb, bm_nkb, bm_batch;
};
// Backward from the stored LSE, bf16 inputs, fp32 gradients, D in {64, 128}.
hipError_t launch_bwd_bf16(const BwdParams &p, hipStream_t stream);
// fp32 path, D in {16, 32, 64, 128, 256}.
hipError_t launch_fwd_f32(const FwdParams &p, hipStream_t stream);

struct BlockMaskParams {
  MaskArgs mask;
  int B, Sq, Skv, q_block, kv_block, nqb, nkb;
  int32_t *num;
  int32_t *idx;
  uint8_t *full;
};
hipError_t launch_block_mask(const BlockMaskParams &p, hipStream_t stream);

struct BlockMaskTransposeParams {
  const int32_t *num, *idx;   // lists by query block [batch, nqb(, nkb)]
  const uint8_t *full;        // may be null
  int32_t *q_num, *q_idx;     // lists by key block [batch, nkb(, nqb)]
  uint8_t *q_full;            // may be null
  int batch, nqb, nkb;
};
hipError_t launch_block_mask_transpose(const BlockMaskTransposeParams &p, hipStream_t stream);

struct DecodeParams {
  const void *q, *k_cache, *v_cache;
  const int32_t *page_table, *seq_lens;
  void *out;
  float *lse;
  int N, Hq, Hkv, D, page_size, max_pages, num_pages;
  float scale;
  MaskArgs mask;   // NONE or SLIDING
  ScoreArgs score;
  float *ws_o;     // [N, Hq, max_splits, D]
  float *ws_lse;   // [N, Hq, max_splits]
  int max_splits;  // split capacity of the workspace per (sequence, head)
};
// Splits per (sequence, head) the workspace must hold: enough for the
// smallest split size the launch may choose.
int decode_max_splits(int max_pages);
// Splits per (sequence, head) the launch for p takes: the workspace needs
// room for this many at least (p's workspace fields are not read).
int decode_launch_splits(const DecodeParams &p);
hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream);

}  // namespace attn
