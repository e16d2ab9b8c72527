"""Paged-KV decode reference and the split/combine identity it rests on.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[FlexAttention page] names PagedAttention in its variant list; [Pallas page]
describes a multi-query paged-attention kernel.  Neither gives a layout; the
one taken here:

* k_cache, v_cache: [num_pages, Hkv, page_size, D]; each (page, kv head) is
  one contiguous page_size x D block;
* page_table: int [N, max_pages]; token t of sequence s lives in page
  page_table[s, t // page_size] at slot t % page_size; entries past
  ceil(L_s / page_size) are never read;
* the single query of sequence s sits at position L_s - 1 and sees every key
  t < L_s; score modifiers use i = L_s - 1;
* with a sliding window (PagedAttention and the sliding window both stand in
  the [FlexAttention page] variant list; the window is that of its §Sliding
  Window + Causal, read as 0 <= i - t < W) the query sees only the keys with
  L_s - W <= t < L_s; the cache slots of the other keys take no part, whatever
  they hold.

Split combine ([Online-Softmax page]: the online-softmax rescaling merges
partial results): with per-range results (O_k normalised, lse_k),
LSE = ln sum_k e^{lse_k} and O = sum_k e^{lse_k - LSE} O_k.
"""

from __future__ import annotations

import numpy as np

from . import attention as _att
from .attention import MaskSpec, ScoreSpec, MASK_NONE, MASK_SLIDING, attention_rows


def gather_paged_kv(k_cache, v_cache, page_table, seq_len: int, s: int):
    """Contiguous K, V [Hkv, L, D] (float64) of sequence s, gathered through
    its page table."""
    k_cache = np.asarray(k_cache)
    page_size = k_cache.shape[2]
    t = np.arange(seq_len)
    pages = np.asarray(page_table)[s, t // page_size]
    slots = t % page_size
    kk = np.asarray(k_cache)[pages, :, slots, :].astype(np.float64)   # [L, Hkv, D]
    vv = np.asarray(v_cache)[pages, :, slots, :].astype(np.float64)
    return kk.transpose(1, 0, 2), vv.transpose(1, 0, 2)


def paged_decode_ref(q, k_cache, v_cache, page_table, seq_lens, scale,
                     score: ScoreSpec = ScoreSpec(), seqs=None, mask: MaskSpec = MaskSpec(MASK_NONE)):
    """Decode attention of one query per sequence over its paged K/V.

    q: [N, Hq, D].  mask: MASK_NONE or MASK_SLIDING (window).  Returns
    (O [N', Hq, D], LSE [N', Hq]) float64 for the sequences in seqs (default
    all).
    """
    if mask.kind not in (MASK_NONE, MASK_SLIDING):
        raise ValueError("paged decode takes no mask or a sliding window")
    q = np.asarray(q)
    n_seq, hq_count, _ = q.shape
    hkv_count = np.asarray(k_cache).shape[1]
    seqs = np.arange(n_seq) if seqs is None else np.asarray(seqs, dtype=np.int64)
    out = np.zeros((len(seqs), hq_count, np.asarray(v_cache).shape[-1]))
    lse = np.zeros((len(seqs), hq_count))
    for si, s in enumerate(seqs):
        length = int(np.asarray(seq_lens)[s])
        if length <= 0:
            # No key at all: the fully-masked-row convention, O = 0 and
            # LSE = -inf.
            out[si] = 0.0
            lse[si] = -np.inf
            continue
        kk, vv = gather_paged_kv(k_cache, v_cache, page_table, length, int(s))
        if mask.kind == MASK_SLIDING:
            # keys before the window are masked below; their slots' contents
            # take no part (zeroed, so that no stored value can leak in)
            t0 = max(0, length - mask.window)
            kk[:, :t0] = 0.0
            vv[:, :t0] = 0.0
        for hq in range(hq_count):
            hkv = _att.kv_head(hq, hq_count, hkv_count)
            o, l = attention_rows(q[s, hq][None, :].astype(np.float64), kk[hkv], vv[hkv],
                                  [length - 1], int(s), hq, hq_count, scale, mask, score)
            out[si, hq] = o[0]
            lse[si, hq] = l[0]
    return out, lse


def split_partials_ref(q_row, k, v, row: int, hq: int, hq_count: int, scale, cuts,
                       score: ScoreSpec = ScoreSpec()):
    """Per-range normalised partial results of one query row.

    cuts: ascending key positions that split 0..m into ranges.  Returns
    (O_parts [n_ranges, D], lse_parts [n_ranges]); an empty range gives O = 0,
    lse = -inf.
    """
    m = np.asarray(k).shape[0]
    bounds = [0] + [int(c) for c in cuts] + [m]
    o_parts, l_parts = [], []
    for a, e in zip(bounds[:-1], bounds[1:]):
        cols = np.arange(a, e)
        if len(cols) == 0:
            o_parts.append(np.zeros(np.asarray(v).shape[-1]))
            l_parts.append(-np.inf)
            continue
        o, l = attention_rows(np.asarray(q_row)[None, :], np.asarray(k)[cols], np.asarray(v)[cols],
                              [row], 0, hq, hq_count, scale, MaskSpec(MASK_NONE), score, col_idx=cols)
        o_parts.append(o[0])
        l_parts.append(l[0])
    return np.array(o_parts), np.array(l_parts)


def lse_combine_ref(o_parts, lse_parts):
    """Merge normalised partials: LSE = ln sum e^{lse_k}, O = sum e^{lse_k-LSE} O_k."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = np.max(lse_parts, axis=0)
    if not np.isfinite(mx).all():
        fin = np.isfinite(mx)
        mx = np.where(fin, mx, 0.0)
    w = np.exp(lse_parts - mx)
    tot = np.sum(w, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(tot > 0, mx + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
        o = np.where(np.expand_dims(tot, -1) > 0,
                     np.tensordot(w, o_parts, axes=(0, 0)) / np.expand_dims(np.where(tot > 0, tot, 1.0), -1),
                     0.0)
    return o, lse
