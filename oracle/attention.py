"""Plain float64 softmax attention with explicit score modifiers and masks.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed, for batch b, query head hq and query row i
([FlexAttention page], §FlexAttention: classic softmax attention, with a
user ``score_mod(score, b, h, q_idx, kv_idx)`` applied to every score before
the softmax):

    hkv       = floor(hq * Hkv / Hq)                      (GQA head map)
    S[i, j]   = s * sum_d Q[b,hq,i,d] * K[b,hkv,j,d]       (s = fp32 scale)
    S[i, j]   = score_mod(S[i, j], hq, i, j)              (score_mod kind:
                S + bias(hq, i, j), or cap * tanh(S / cap))
    S[i, j]   = -inf where not visible(b, i, j)           (mask kind)
    P[i, :]   = softmax(S[i, :])                          (3-pass safe form)
    O[i, :]   = sum_j P[i, j] * V[b,hkv,j,:]
    LSE[i]    = m_i + ln l_i   (natural log; m_i row max, l_i = sum e^{S-m_i})

A row with no visible key has O = 0 and LSE = -inf.

Readings taken where the pages are silent (their formulas were images):
* the scale is applied before the bias (score_mod sees scaled scores);
* ALiBi adds slope_hq * (j - i), slope_h = 2^(-8 (h+1) / Hq), h the 0-based
  query head (the variant is only named in the page's list);
* relative position adds c * (i - j) (§相对位置编码: the score is adjusted by
  the query-key distance; c is a per-call constant, default 1);
* soft-capping maps the scaled score x to cap * tanh(x / cap), cap > 0 a
  per-call constant (§Soft-capping names the technique, used by Gemma 2 and
  Grok-1, but its formula did not survive; this is the usual definition: a
  smooth, odd, increasing squashing of every score into (-cap, cap) that is
  the identity to first order);
* causal is inclusive, j <= i (§Causal Mask: each token attends to the tokens
  before it; row 0 then returns V[0]);
* the sliding window keeps exactly W keys, self included: 0 <= i - j < W
  (§Sliding Window + Causal: the most recent 1024 tokens, with causal);
* PrefixLM: j <= i or j < P (named only in the variant list);
* document mask: doc[b, i] == doc[b, j] and j <= i (named only in the list);
* AND-composition: a key is visible when every listed kind's predicate holds,
  each with the spec's own window / prefix / document ids (the variant list
  names the combination sliding window + document + causal; combining masks
  is read as intersecting them, the plain reading of "+" for restrictions);
* indices are raw row/column numbers, as in the page's score_mod loop.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_SLIDING = 2       # causal + window
MASK_PREFIX_LM = 3
MASK_DOCUMENT = 4      # causal within a document
MASK_AND = 5           # conjunction of the kinds in MaskSpec.and_kinds

SCORE_NONE = 0
SCORE_ALIBI = 1
SCORE_REL_POS = 2
SCORE_SOFTCAP = 3


@dataclass(frozen=True)
class MaskSpec:
    kind: int = MASK_NONE
    window: int = 0
    prefix_len: int = 0
    doc_ids: Optional[np.ndarray] = None  # int [B, S] (query and key share it)
    and_kinds: Tuple[int, ...] = ()       # MASK_AND: the kinds intersected


@dataclass(frozen=True)
class ScoreSpec:
    kind: int = SCORE_NONE
    slopes: Optional[np.ndarray] = None   # [Hq]; None -> alibi_slopes(Hq)
    rel_scale: float = 1.0
    softcap: float = 0.0                  # SOFTCAP: the cap, > 0


def alibi_slopes(hq_count: int) -> np.ndarray:
    """ALiBi head slopes 2^(-8 (h+1) / Hq), h = 0..Hq-1, in float64."""
    h = np.arange(hq_count, dtype=np.float64)
    return np.exp2(-8.0 * (h + 1.0) / hq_count)


def visible(mask: MaskSpec, b: int, i, j) -> np.ndarray:
    """Boolean visibility of key j to query i (broadcast to [len(i), len(j)]).

    [FlexAttention page]: §Causal Mask, §Sliding Window + Causal, and the
    PrefixLM / document-mask entries of the variant list.
    """
    i = np.asarray(i, dtype=np.int64)[:, None]
    j = np.asarray(j, dtype=np.int64)[None, :]
    kind = mask.kind
    if kind == MASK_NONE:
        return np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if kind == MASK_CAUSAL:
        return j <= i
    if kind == MASK_SLIDING:
        d = i - j
        return (d >= 0) & (d < mask.window)
    if kind == MASK_PREFIX_LM:
        return (j <= i) | (j < mask.prefix_len)
    if kind == MASK_DOCUMENT:
        doc = np.asarray(mask.doc_ids)[b]
        return (doc[i] == doc[j]) & (j <= i)
    if kind == MASK_AND:
        out = np.ones((i.shape[0], j.shape[1]), dtype=bool)
        for part in mask.and_kinds:
            if part == MASK_AND:
                raise ValueError("AND terms are plain kinds")
            out &= visible(replace(mask, kind=part, and_kinds=()), b, i[:, 0], j[0, :])
        return out
    raise ValueError(f"unknown mask kind {kind}")


def bias(score: ScoreSpec, hq: int, hq_count: int, i, j):
    """Additive score modifier for query head hq at positions (i, j).

    [FlexAttention page] §相对位置编码 (bias from the distance, never stored
    as an S x S tensor by the kernel) and the ALiBi entry of the variant list.
    Returns a scalar 0.0 for the identity modifier (§全注意力).
    """
    if score.kind == SCORE_NONE:
        return 0.0
    i = np.asarray(i, dtype=np.float64)[:, None]
    j = np.asarray(j, dtype=np.float64)[None, :]
    if score.kind == SCORE_ALIBI:
        slopes = alibi_slopes(hq_count) if score.slopes is None else np.asarray(score.slopes, np.float64)
        return slopes[hq] * (j - i)
    if score.kind == SCORE_REL_POS:
        return float(score.rel_scale) * (i - j)
    if score.kind == SCORE_SOFTCAP:
        raise ValueError("soft-capping is not an additive bias")
    raise ValueError(f"unknown score kind {score.kind}")


def score_mod(score: ScoreSpec, s, hq: int, hq_count: int, i, j) -> np.ndarray:
    """The modified scores score_mod(S) of a block S[len(i), len(j)].

    [FlexAttention page] §FlexAttention (every score passes through score_mod
    before the softmax).  Additive kinds add bias(); SOFTCAP returns
    cap * tanh(S / cap) (§Soft-capping).
    """
    if score.kind == SCORE_SOFTCAP:
        cap = float(score.softcap)
        if not cap > 0.0:
            raise ValueError("soft-capping needs cap > 0")
        return cap * np.tanh(np.asarray(s, dtype=np.float64) / cap)
    return s + bias(score, hq, hq_count, i, j)


def kv_head(hq: int, hq_count: int, hkv_count: int) -> int:
    """GQA head map: consecutive groups of Hq/Hkv query heads share a kv head."""
    return (hq * hkv_count) // hq_count


def _fp32_scale(scale: float) -> float:
    # The library takes the scale as a float32 argument; the oracle uses that
    # exact value, upcast, so both sides scale by the same number.
    return float(np.float32(scale))


def scores_block(q_rows, k, scale, mask: MaskSpec, score: ScoreSpec,
                 b: int, hq: int, hq_count: int, row_idx, col_idx=None) -> np.ndarray:
    """Materialised modified scores S[i, j] for the given query rows.

    q_rows: [n, D] (rows row_idx of Q[b, hq]); k: [m, D] (keys col_idx).
    Order: scale, then score_mod, then mask (-inf where not visible).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    row_idx = np.asarray(row_idx, dtype=np.int64)
    col_idx = np.arange(k.shape[0]) if col_idx is None else np.asarray(col_idx, np.int64)
    s = _fp32_scale(scale) * (q_rows @ k.T)
    s = score_mod(score, s, hq, hq_count, row_idx, col_idx)
    vis = visible(mask, b, row_idx, col_idx)
    return np.where(vis, s, -np.inf)


def softmax_safe3(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """3-pass safe softmax over the last axis ([Online-Softmax page] abstract).

    Pass 1: row max m.  Pass 2: l = sum e^{s - m}.  Pass 3: P = e^{s - m} / l.
    Rows that are entirely -inf give m = -inf, l = 0 and P = 0.
    Returns (P, m, l).
    """
    m = np.max(s, axis=-1)
    m_shift = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_shift[..., None])
    l = np.sum(e, axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l[..., None] > 0, e / np.where(l > 0, l, 1.0)[..., None], 0.0)
    return p, m, l


def softmax_online2(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """2-pass online softmax ([Online-Softmax page] abstract).

    Pass 1 walks the columns once keeping a running max m and a running sum l
    that is rescaled by e^{m_old - m_new} whenever the max grows.  Pass 2
    normalises.  Returns (P, m, l) like softmax_safe3.
    """
    s = np.asarray(s, dtype=np.float64)
    n, cols = s.shape
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    for j in range(cols):
        m_new = np.maximum(m, s[:, j])
        fin = np.isfinite(m_new)
        base = np.where(fin, m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
        l = l * alpha + np.exp(s[:, j] - base)
        m = m_new
    m_shift = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(l[:, None] > 0, np.exp(s - m_shift[:, None]) / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return p, m, l


def softmax_naive(s: np.ndarray) -> np.ndarray:
    """Textbook e^{s} / sum e^{s}; valid only where e^{s} cannot overflow."""
    e = np.exp(np.asarray(s, dtype=np.float64))
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_rows(q_rows, k, v, row_idx, b: int, hq: int, hq_count: int, scale,
                   mask: MaskSpec = MaskSpec(), score: ScoreSpec = ScoreSpec(),
                   col_idx=None) -> Tuple[np.ndarray, np.ndarray]:
    """O and LSE for some query rows of one (b, hq) against keys k, values v.

    k, v: [m, D] for key positions col_idx (default 0..m-1).  Returns
    (O [n, Dv], LSE [n]) in float64.  The plain definition: materialised
    scores, 3-pass safe softmax, dense P @ V.
    """
    s = scores_block(q_rows, k, scale, mask, score, b, hq, hq_count, row_idx, col_idx)
    p, m, l = softmax_safe3(s)
    o = p @ np.asarray(v, dtype=np.float64)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def attention_ref(q, k, v, scale, mask: MaskSpec = MaskSpec(), score: ScoreSpec = ScoreSpec(),
                  rows=None, heads=None, batches=None, row_block: int = 1024):
    """Full attention forward, float64, layout Q/O [B,Hq,Sq,D], K/V [B,Hkv,Skv,D].

    rows / heads / batches optionally restrict the computation to a subset
    (used to check sampled outputs at sizes where the full result would take
    too long on the CPU); the result then has those subsets as its axes.
    Returns (O, LSE) with LSE [B', Hq', n].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    bsz, hq_count, sq, _ = q.shape
    hkv_count = k.shape[1]
    if hq_count % hkv_count != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    rows = np.arange(sq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(hq_count) if heads is None else np.asarray(heads, dtype=np.int64)
    batches = np.arange(bsz) if batches is None else np.asarray(batches, dtype=np.int64)
    dv = v.shape[-1]
    out = np.zeros((len(batches), len(heads), len(rows), dv))
    lse = np.zeros((len(batches), len(heads), len(rows)))
    for bi, b in enumerate(batches):
        for hi, hq in enumerate(heads):
            hkv = kv_head(int(hq), hq_count, hkv_count)
            kk = k[b, hkv].astype(np.float64)
            vv = v[b, hkv].astype(np.float64)
            for r0 in range(0, len(rows), row_block):
                ridx = rows[r0:r0 + row_block]
                o_blk, l_blk = attention_rows(q[b, hq][ridx], kk, vv, ridx, int(b), int(hq),
                                              hq_count, scale, mask, score)
                out[bi, hi, r0:r0 + len(ridx)] = o_blk
                lse[bi, hi, r0:r0 + len(ridx)] = l_blk
    return out, lse


def attention_bruteforce(q, k, v, scale, mask: MaskSpec = MaskSpec(),
                         score: ScoreSpec = ScoreSpec()):
    """Scalar-loop form for tiny shapes: the page's five-deep score_mod loop.

    [FlexAttention page] §FlexAttention: for every (b, h, q_idx, kv_idx) the
    modified score is score_mod(score, b, h, q_idx, kv_idx).  Everything here
    is pure Python floats (math.exp / math.log), one element at a time, with
    no NumPy arithmetic, so it checks the vectorised form independently.
    """
    q = np.asarray(q, dtype=np.float64).tolist()
    k = np.asarray(k, dtype=np.float64).tolist()
    v = np.asarray(v, dtype=np.float64).tolist()
    bsz, hq_count, sq = len(q), len(q[0]), len(q[0][0])
    hkv_count, skv = len(k[0]), len(k[0][0])
    d = len(q[0][0][0])
    dv = len(v[0][0][0])
    s_fp = float(np.float32(scale))      # the float32 argument, upcast
    slopes = None
    if score.kind == SCORE_ALIBI:
        if score.slopes is None:
            slopes = [2.0 ** (-8.0 * (h + 1) / hq_count) for h in range(hq_count)]
        else:
            slopes = [float(x) for x in score.slopes]
    doc = None if mask.doc_ids is None else np.asarray(mask.doc_ids).tolist()

    def score_mod_1(x, b, h, qi, kj):
        if score.kind == SCORE_ALIBI:
            x = x + slopes[h] * (kj - qi)
        elif score.kind == SCORE_REL_POS:
            x = x + float(score.rel_scale) * (qi - kj)
        elif score.kind == SCORE_SOFTCAP:
            x = float(score.softcap) * math.tanh(x / float(score.softcap))
        return x

    def is_visible(b, qi, kj, kind=mask.kind):
        if kind == MASK_NONE:
            return True
        if kind == MASK_CAUSAL:
            return kj <= qi
        if kind == MASK_SLIDING:
            return 0 <= qi - kj < mask.window
        if kind == MASK_PREFIX_LM:
            return kj <= qi or kj < mask.prefix_len
        if kind == MASK_DOCUMENT:
            return doc[b][qi] == doc[b][kj] and kj <= qi
        if kind == MASK_AND:
            return all(is_visible(b, qi, kj, part) for part in mask.and_kinds)
        raise ValueError(kind)

    out = [[[[0.0] * dv for _ in range(sq)] for _ in range(hq_count)] for _ in range(bsz)]
    lse = [[[0.0] * sq for _ in range(hq_count)] for _ in range(bsz)]
    for b in range(bsz):
        for h in range(hq_count):
            g = (h * hkv_count) // hq_count
            for qi in range(sq):
                row = []
                for kj in range(skv):
                    dot = 0.0
                    for t in range(d):
                        dot += q[b][h][qi][t] * k[b][g][kj][t]
                    x = score_mod_1(s_fp * dot, b, h, qi, kj)
                    row.append(x if is_visible(b, qi, kj) else None)
                live = [x for x in row if x is not None]
                if not live:
                    lse[b][h][qi] = -math.inf
                    continue
                mx = max(live)
                w = [0.0 if x is None else math.exp(x - mx) for x in row]
                tot = sum(w)
                for t in range(dv):
                    acc = 0.0
                    for kj in range(skv):
                        acc += w[kj] * v[b][g][kj][t]
                    out[b][h][qi][t] = acc / tot
                lse[b][h][qi] = mx + math.log(tot)
    return np.array(out, dtype=np.float64), np.array(lse, dtype=np.float64)


def attention_one_pass(q, k, v, scale, mask: MaskSpec = MaskSpec(),
                       score: ScoreSpec = ScoreSpec(), kv_tile: int = 16):
    """1-pass FlashAttention recurrence in float64 ([Online-Softmax page]).

    Keys are consumed tile by tile; per query row a running max m, a running
    sum l and an unnormalised output acc are rescaled by e^{m_old - m_new}
    when the max grows, and O = acc / l, LSE = m + ln l at the end.  A
    cross-check of the 3-pass form, not the oracle's primary definition.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, hq_count, sq, _ = q.shape
    hkv_count, skv = k.shape[1], k.shape[2]
    out = np.zeros(q.shape[:3] + (v.shape[-1],))
    lse = np.zeros(q.shape[:3])
    rows = np.arange(sq)
    for b in range(bsz):
        for hq in range(hq_count):
            hkv = kv_head(hq, hq_count, hkv_count)
            m = np.full(sq, -np.inf)
            l = np.zeros(sq)
            acc = np.zeros((sq, v.shape[-1]))
            for j0 in range(0, skv, kv_tile):
                cols = np.arange(j0, min(skv, j0 + kv_tile))
                s = scores_block(q[b, hq], k[b, hkv, cols], scale, mask, score, b, hq,
                                 hq_count, rows, cols)
                m_new = np.maximum(m, np.max(s, axis=1))
                fin = np.isfinite(m_new)
                base = np.where(fin, m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
                p = np.exp(s - base[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, hkv, cols]
                m = m_new
            with np.errstate(divide="ignore", invalid="ignore"):
                out[b, hq] = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
                lse[b, hq] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse
