"""Pins of the BlockMask and paged-decode parts of the oracle.

BlockMask: the vectorised builder against an element-by-element scalar scan,
and against closed-form block counts for causal and sliding-window masks and
an interval-arithmetic count for document masks (worked out from document
boundaries, never from the element grid).

Paged decode: against a contiguous-K/V attention built by an explicit
token-by-token gather in the test, and the split/combine identity of the
online-softmax merge.
"""

import math

import numpy as np
import pytest

import oracle
import workloads
from oracle import MaskSpec, ScoreSpec, MASK_NONE, MASK_CAUSAL, MASK_SLIDING, MASK_PREFIX_LM, \
    MASK_DOCUMENT, MASK_AND, SCORE_NONE, SCORE_ALIBI, SCORE_REL_POS


def _ids(lengths, batch=1):
    return np.tile(np.repeat(np.arange(len(lengths)), lengths)[None, :], (batch, 1))


CASES = [
    (MaskSpec(MASK_NONE), 2, 23, 23, 4, 8),
    (MaskSpec(MASK_CAUSAL), 1, 37, 37, 8, 8),
    (MaskSpec(MASK_CAUSAL), 1, 20, 33, 8, 4),
    (MaskSpec(MASK_SLIDING, window=5), 1, 41, 41, 8, 8),
    (MaskSpec(MASK_SLIDING, window=17), 2, 40, 40, 8, 16),
    (MaskSpec(MASK_PREFIX_LM, prefix_len=11), 1, 30, 30, 8, 8),
    (MaskSpec(MASK_DOCUMENT, doc_ids=_ids([7, 3, 12, 9, 2], 2)), 2, 33, 33, 8, 8),
    (MaskSpec(MASK_AND, window=6, doc_ids=_ids([7, 3, 12, 9, 2], 2),
              and_kinds=(MASK_SLIDING, MASK_DOCUMENT)), 2, 33, 33, 8, 4),
    (MaskSpec(MASK_AND, window=11, prefix_len=9, doc_ids=_ids([20, 13], 1),
              and_kinds=(MASK_CAUSAL, MASK_SLIDING, MASK_DOCUMENT, MASK_PREFIX_LM)), 1, 33, 33, 4, 8),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_block_mask_matches_scalar_scan(ci):
    mask, b, sq, skv, qb, kb = CASES[ci]
    got = oracle.block_mask_ref(mask, b, sq, skv, qb, kb)
    want = oracle.block_mask_bruteforce(mask.kind, b, sq, skv, qb, kb, mask.window, mask.prefix_len,
                                        mask.doc_ids, mask.and_kinds)
    for g, w in zip(got, want):
        assert g.dtype == w.dtype and g.shape == w.shape
        assert np.array_equal(g, w)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_block_mask_cols_are_the_transposed_incidence(ci):
    # per key block, the query blocks whose row list holds it, same full flag;
    # checked against the scalar scan's row lists
    mask, b, sq, skv, qb, kb = CASES[ci]
    rnum, ridx, rfull = oracle.block_mask_bruteforce(mask.kind, b, sq, skv, qb, kb, mask.window,
                                                     mask.prefix_len, mask.doc_ids, mask.and_kinds)
    cnum, cidx, cfull = oracle.block_mask_cols_ref(mask, b, sq, skv, qb, kb)
    nqb, nkb = rnum.shape[2], cnum.shape[2]
    for bb in range(b):
        inc = {}
        for q in range(nqb):
            for n in range(rnum[bb, 0, q]):
                inc[(q, int(ridx[bb, 0, q, n]))] = int(rfull[bb, 0, q, n])
        for k in range(nkb):
            want = sorted(q for (q, kk) in inc if kk == k)
            got = [int(x) for x in cidx[bb, 0, k, :cnum[bb, 0, k]]]
            assert got == want
            assert [int(x) for x in cfull[bb, 0, k, :len(want)]] == [inc[(q, k)] for q in want]
            assert np.all(cidx[bb, 0, k, len(want):] == -1) and np.all(cfull[bb, 0, k, len(want):] == 0)


def test_block_mask_cols_causal_closed_form():
    # causal, 16 x 16 blocks: key block kb is seen by query blocks kb..15,
    # fully by kb+1..15
    num, idx, full = oracle.block_mask_cols_ref(MaskSpec(MASK_CAUSAL), 1, 2048, 2048, 128, 128)
    for kb in range(16):
        assert num[0, 0, kb] == 16 - kb
        assert list(idx[0, 0, kb, :16 - kb]) == list(range(kb, 16))
        assert list(full[0, 0, kb, :16 - kb]) == [0] + [1] * (15 - kb)


def test_block_mask_causal_counts_closed_form():
    num, idx, full = oracle.block_mask_ref(MaskSpec(MASK_CAUSAL), 1, 2048, 2048, 128, 128)
    n = 2048 // 128
    assert int(num.sum()) == n * (n + 1) // 2 == 136
    assert int(full.sum()) == n * (n - 1) // 2 == 120
    for qb in range(n):
        assert list(idx[0, 0, qb, :qb + 1]) == list(range(qb + 1))
        assert list(full[0, 0, qb, :qb + 1]) == [1] * qb + [0]


def test_block_mask_window_counts_closed_form():
    # rows 128qb..128qb+127, cols 128kb..: listed iff the distance range
    # [128(qb-kb)-127, 128(qb-kb)+127] meets [0, W); full iff it lies inside.
    s, w, blk = 8192, 1024, 128
    n = s // blk
    num, idx, full = oracle.block_mask_ref(MaskSpec(MASK_SLIDING, window=w), 1, s, s, blk, blk)
    # listed: 128t - 127 < W  ->  t <= (W + blk - 2) // blk;  full: 1 <= t and 128t + 127 < W
    listed = sum(min(qb + 1, (w + blk - 2) // blk + 1) for qb in range(n))
    n_full = sum(min(qb, (w - blk) // blk) for qb in range(n))
    assert int(num.sum()) == listed == 540
    assert int(full.sum()) == n_full == 420


def _doc_interval_counts(lengths, blk):
    """Listed / full block counts of a causal document mask from document
    intervals alone."""
    bounds = np.cumsum([0] + list(lengths))
    s = int(bounds[-1])
    n = -(-s // blk)
    listed = full = 0
    for qb in range(n):
        q0, q1 = qb * blk, min(s, (qb + 1) * blk) - 1
        for kb in range(n):
            k0, k1 = kb * blk, min(s, (kb + 1) * blk) - 1
            hit = False
            for a, e in zip(bounds[:-1], bounds[1:]):
                lo_q, hi_q = max(a, q0), min(e - 1, q1)
                lo_k, hi_k = max(a, k0), min(e - 1, k1)
                if lo_q <= hi_q and lo_k <= hi_k and lo_k <= hi_q:
                    hit = True
            if hit:
                listed += 1
                same = any(a <= min(q0, k0) and max(q1, k1) <= e - 1 for a, e in zip(bounds[:-1], bounds[1:]))
                if same and k1 <= q0:
                    full += 1
    return listed, full


def test_block_mask_document_counts_seed0():
    lengths = workloads.doc_lengths(16384, 256, 4096, seed=0)
    assert lengths == [3523, 2702, 2219, 1292, 1438, 413, 544, 319, 929, 3005]
    num, idx, full = oracle.block_mask_ref(MaskSpec(MASK_DOCUMENT, doc_ids=_ids(lengths)), 1, 16384,
                                           16384, 128, 128)
    listed, n_full = _doc_interval_counts(lengths, 128)
    assert (int(num.sum()), int(full.sum())) == (listed, n_full) == (1348, 1024)


def test_block_mask_document_counts_ragged():
    lengths = [100, 37, 250, 1, 60]
    num, _, full = oracle.block_mask_ref(MaskSpec(MASK_DOCUMENT, doc_ids=_ids(lengths)), 1, 448, 448, 64, 64)
    assert (int(num.sum()), int(full.sum())) == _doc_interval_counts(lengths, 64)


def test_block_mask_tail_padding():
    num, idx, full = oracle.block_mask_ref(MaskSpec(MASK_CAUSAL), 1, 300, 300, 128, 128)
    assert num.tolist() == [[[1, 2, 3]]]
    assert idx[0, 0, 0].tolist() == [0, -1, -1]
    assert full[0, 0, 1].tolist() == [1, 0, 0]
    # the clipped last block (rows 256..299, cols 256..299) is not full
    assert full[0, 0, 2].tolist() == [1, 1, 0]


# ----------------------------------------------------------------------------
# paged decode

def _small_paged(seed=0, n=5, hq=8, hkv=2, d=16, page=4, max_pages=12):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, page * max_pages, size=n, endpoint=True)
    pages = [-(-int(L) // page) for L in lengths]
    pool = sum(pages) + 3
    perm = rng.permutation(pool)
    table = np.full((n, max_pages), -1, dtype=np.int64)
    pos = 0
    for s, c in enumerate(pages):
        table[s, :c] = perm[pos:pos + c]
        pos += c
    q = rng.standard_normal((n, hq, d))
    kc = rng.standard_normal((pool, hkv, page, d))
    vc = rng.standard_normal((pool, hkv, page, d))
    return q, kc, vc, table, lengths


@pytest.mark.parametrize("score", [ScoreSpec(SCORE_NONE), ScoreSpec(SCORE_ALIBI),
                                   ScoreSpec(SCORE_REL_POS, rel_scale=-0.1)])
def test_paged_decode_equals_contiguous_attention(score):
    q, kc, vc, table, lengths = _small_paged()
    n, hq, d = q.shape
    hkv, page = kc.shape[1], kc.shape[2]
    o, lse = oracle.paged_decode_ref(q, kc, vc, table, lengths, 0.25, score)
    for s in range(n):
        L = int(lengths[s])
        kk = np.zeros((1, hkv, L, d))
        vv = np.zeros((1, hkv, L, d))
        for t in range(L):                       # token-by-token gather
            p = table[s, t // page]
            kk[0, :, t] = kc[p, :, t % page]
            vv[0, :, t] = vc[p, :, t % page]
        qq = np.zeros((1, hq, L, d))
        qq[0, :, L - 1] = q[s]
        # the decode query sits at position L-1 and sees every key t < L
        oc, lc = oracle.attention_ref(qq, kk, vv, 0.25, MaskSpec(MASK_CAUSAL), score, rows=[L - 1])
        np.testing.assert_allclose(o[s], oc[0, :, 0], atol=1e-13)
        np.testing.assert_allclose(lse[s], lc[0, :, 0], atol=1e-13)


def test_paged_decode_ignores_unused_slots():
    q, kc, vc, table, lengths = _small_paged(seed=3)
    o1, l1 = oracle.paged_decode_ref(q, kc, vc, table, lengths, 0.3)
    kc2, vc2 = kc.copy(), vc.copy()
    used = set()
    for s, L in enumerate(lengths):
        for t in range(int(L)):
            used.add((int(table[s, t // 4]), t % 4))
    for p in range(kc.shape[0]):
        for slot in range(4):
            if (p, slot) not in used:
                kc2[p, :, slot] = np.nan
                vc2[p, :, slot] = np.nan
    o2, l2 = oracle.paged_decode_ref(q, kc2, vc2, table, lengths, 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_split_combine_equals_unsplit():
    rng = np.random.default_rng(8)
    m, d = 200, 16
    q, k, v = rng.standard_normal(d), rng.standard_normal((m, d)), rng.standard_normal((m, d))
    for score in (ScoreSpec(SCORE_NONE), ScoreSpec(SCORE_ALIBI)):
        o_full, l_full = oracle.attention_rows(q[None], k, v, [m - 1], 0, 3, 8, 0.5,
                                               MaskSpec(MASK_NONE), score)
        for cuts in ([100], [1, 2, 3, 150], [0, 0, 64, 128, 192], sorted(rng.integers(0, m, 7))):
            op, lp = oracle.split_partials_ref(q, k, v, m - 1, 3, 8, 0.5, cuts, score)
            oc, lc = oracle.lse_combine_ref(op, lp)
            np.testing.assert_allclose(oc, o_full[0], atol=1e-14)
            assert lc == pytest.approx(l_full[0], abs=1e-13)


def test_paged_decode_empty_sequence():
    # A sequence with no token has no key to attend to: the fully masked row
    # convention (O = 0, LSE = -inf), and the other sequences are unaffected.
    q, kc, vc, table, lengths = _small_paged(seed=5)
    lengths2 = np.array(lengths).copy()
    lengths2[1] = 0
    o1, l1 = oracle.paged_decode_ref(q, kc, vc, table, lengths, 0.3)
    o2, l2 = oracle.paged_decode_ref(q, kc, vc, table, lengths2, 0.3)
    assert np.all(o2[1] == 0.0) and np.all(l2[1] == -np.inf)
    keep = [s for s in range(len(lengths)) if s != 1]
    assert np.array_equal(o1[keep], o2[keep]) and np.array_equal(l1[keep], l2[keep])


@pytest.mark.parametrize("window", [1, 3, 4, 5, 17, 1000])
def test_paged_decode_sliding_window(window):
    # Windowed decode equals contiguous attention of the query row L-1 under
    # the sliding-window mask, computed token by token.
    q, kc, vc, table, lengths = _small_paged(seed=6)
    n, hq, d = q.shape
    hkv, page = kc.shape[1], kc.shape[2]
    ms = MaskSpec(MASK_SLIDING, window=window)
    score = ScoreSpec(SCORE_ALIBI)
    o, lse = oracle.paged_decode_ref(q, kc, vc, table, lengths, 0.25, score, mask=ms)
    for s in range(n):
        L = int(lengths[s])
        kk = np.zeros((1, hkv, L, d))
        vv = np.zeros((1, hkv, L, d))
        for t in range(L):
            p = table[s, t // page]
            kk[0, :, t] = kc[p, :, t % page]
            vv[0, :, t] = vc[p, :, t % page]
        qq = np.zeros((1, hq, L, d))
        qq[0, :, L - 1] = q[s]
        oc, lc = oracle.attention_ref(qq, kk, vv, 0.25, ms, score, rows=[L - 1])
        np.testing.assert_allclose(o[s], oc[0, :, 0], atol=1e-13)
        np.testing.assert_allclose(lse[s], lc[0, :, 0], atol=1e-13)


def test_paged_decode_window_closed_forms():
    q, kc, vc, table, lengths = _small_paged(seed=7)
    page = kc.shape[2]
    # window 1: the query sees only its own key, O = V[L-1], LSE = its score
    o1, l1 = oracle.paged_decode_ref(q, kc, vc, table, lengths, 0.3, mask=MaskSpec(MASK_SLIDING, window=1))
    for s, L in enumerate(lengths):
        p = table[s, (int(L) - 1) // page]
        np.testing.assert_allclose(o1[s], vc[p, :, (int(L) - 1) % page].repeat(4, axis=0), atol=1e-13)
        kv = kc[p, :, (int(L) - 1) % page].repeat(4, axis=0)
        np.testing.assert_allclose(l1[s], 0.3 * np.sum(q[s] * kv, axis=-1), atol=1e-12)
    # a window at least as long as every sequence: no window
    o2, l2 = oracle.paged_decode_ref(q, kc, vc, table, lengths, 0.3,
                                     mask=MaskSpec(MASK_SLIDING, window=int(max(lengths))))
    o3, l3 = oracle.paged_decode_ref(q, kc, vc, table, lengths, 0.3)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)
    # slots before the window take no part, whatever they hold
    kc2, vc2 = kc.copy(), vc.copy()
    for s, L in enumerate(lengths):
        for t in range(max(0, int(L) - 3)):
            kc2[table[s, t // page], :, t % page] = np.nan
            vc2[table[s, t // page], :, t % page] = np.nan
    o4, l4 = oracle.paged_decode_ref(q, kc2, vc2, table, lengths, 0.3, mask=MaskSpec(MASK_SLIDING, window=3))
    o5, l5 = oracle.paged_decode_ref(q, kc, vc, table, lengths, 0.3, mask=MaskSpec(MASK_SLIDING, window=3))
    assert np.array_equal(o4, o5) and np.array_equal(l4, l5)
