"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check below ties the oracle to something other than itself: the pages'
scalar score_mod loop (brute force), the agreement of the three softmax forms
named by the Online-Softmax article, closed forms that hold for special inputs
(Q = 0, K = 0, constant V, scale = 0), invariances (key permutation, per-row
shift, GQA as repeated heads) and an independent library routine (torch's CPU
scaled_dot_product_attention in float64).  test_oracle_mutations.py plants
plausible mistakes in the oracle and checks that these pins catch them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as att
from oracle import (MaskSpec, ScoreSpec, MASK_NONE, MASK_CAUSAL, MASK_SLIDING,
                    MASK_PREFIX_LM, MASK_DOCUMENT, SCORE_NONE, SCORE_ALIBI, SCORE_REL_POS,
                    SCORE_SOFTCAP, MASK_AND)

RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def doc_ids_for(lengths, batch=1):
    return np.tile(np.repeat(np.arange(len(lengths)), lengths)[None, :], (batch, 1))


def all_masks(s, lengths=None):
    lengths = lengths or [3, 5, s - 8]
    return [
        MaskSpec(MASK_NONE),
        MaskSpec(MASK_CAUSAL),
        MaskSpec(MASK_SLIDING, window=4),
        MaskSpec(MASK_PREFIX_LM, prefix_len=5),
        MaskSpec(MASK_DOCUMENT, doc_ids=doc_ids_for(lengths, 2)),
        # sliding window + document + causal, intersected
        MaskSpec(MASK_AND, window=4, doc_ids=doc_ids_for(lengths, 2),
                 and_kinds=(MASK_SLIDING, MASK_DOCUMENT, MASK_CAUSAL)),
    ]


N_MASKS = 6


ALL_SCORES = [ScoreSpec(SCORE_NONE), ScoreSpec(SCORE_ALIBI), ScoreSpec(SCORE_REL_POS, rel_scale=-0.3)]
# every modifier kind: the additive ones above and soft-capping
ALL_MODS = ALL_SCORES + [ScoreSpec(SCORE_SOFTCAP, softcap=0.75)]


# ----------------------------------------------------------------------------
# softmax forms (Online-Softmax article, abstract)

def check_softmax_forms():
    s = rand(7, 33) * 3.0
    s[2, 5:] = -np.inf
    s[4, :] = -np.inf                       # a fully masked row
    p3, m3, l3 = att.softmax_safe3(s)
    p2, m2, l2 = att.softmax_online2(s)
    np.testing.assert_allclose(p3, p2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(m3[np.isfinite(m3)], m2[np.isfinite(m2)], rtol=0, atol=0)
    np.testing.assert_allclose(l3, l2, rtol=1e-13, atol=0)
    live = np.isfinite(m3)
    pn = att.softmax_naive(s[live])
    np.testing.assert_allclose(p3[live], pn, rtol=0, atol=1e-14)
    np.testing.assert_allclose(p3[live].sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p3[~live] == 0.0)
    # the max-shifted form must be safe where the naive one overflows
    big = np.array([[1000.0, 999.0, 998.0]])
    pb, mb, lb = att.softmax_safe3(big)
    e = np.array([1.0, math.exp(-1.0), math.exp(-2.0)])
    np.testing.assert_allclose(pb[0], e / e.sum(), rtol=1e-15)
    assert mb[0] == 1000.0


def test_softmax_forms_agree():
    check_softmax_forms()


# ----------------------------------------------------------------------------
# brute force: the pages' scalar score_mod loop on tiny shapes

def check_bruteforce(mask, score, seed=0):
    rng = np.random.default_rng(seed)
    b, hq, hkv, s, d = 2, 4, 2, 16, 8
    q, k, v = rand(b, hq, s, d, rng=rng), rand(b, hkv, s, d, rng=rng), rand(b, hkv, s, d, rng=rng)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref = oracle.attention_ref(q, k, v, scale, mask, score)
    o_bf, l_bf = oracle.attention_bruteforce(q, k, v, scale, mask, score)
    np.testing.assert_allclose(o_ref, o_bf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_ref, l_bf, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mi", range(N_MASKS))
@pytest.mark.parametrize("si", range(4))
def test_bruteforce_matches_vectorised(mi, si):
    check_bruteforce(all_masks(16)[mi], ALL_MODS[si], seed=10 * mi + si)


def test_bruteforce_rectangular_none_mask():
    rng = np.random.default_rng(5)
    q, k, v = rand(1, 2, 5, 4, rng=rng), rand(1, 1, 9, 4, rng=rng), rand(1, 1, 9, 3, rng=rng)
    o_ref, l_ref = oracle.attention_ref(q, k, v, 0.7, MaskSpec(MASK_NONE), ScoreSpec(SCORE_ALIBI))
    o_bf, l_bf = oracle.attention_bruteforce(q, k, v, 0.7, MaskSpec(MASK_NONE), ScoreSpec(SCORE_ALIBI))
    np.testing.assert_allclose(o_ref, o_bf, atol=1e-12)
    np.testing.assert_allclose(l_ref, l_bf, atol=1e-12)


# ----------------------------------------------------------------------------
# 1-pass recurrence (FlashAttention form) equals the 3-pass definition

@pytest.mark.parametrize("mi", range(N_MASKS))
def test_one_pass_matches_three_pass(mi):
    rng = np.random.default_rng(77 + mi)
    b, hq, hkv, s, d = 2, 4, 2, 37, 8
    q, k, v = rand(b, hq, s, d, rng=rng), rand(b, hkv, s, d, rng=rng), rand(b, hkv, s, d, rng=rng)
    mask = all_masks(s, [10, 20, 7])[mi]
    for score in ALL_MODS:
        o3, l3 = oracle.attention_ref(q, k, v, 0.4, mask, score)
        o1, l1 = oracle.attention_one_pass(q, k, v, 0.4, mask, score, kv_tile=8)
        np.testing.assert_allclose(o1, o3, atol=1e-13)
        np.testing.assert_allclose(l1, l3, atol=1e-13)


# ----------------------------------------------------------------------------
# library cross-check: torch CPU SDPA (PyTorch 2.0 page), float64

def check_against_torch_sdpa(mask, score, seed=3):
    rng = np.random.default_rng(seed)
    b, hq, hkv, s, d = 2, 4, 2, 24, 16
    q, k, v = rand(b, hq, s, d, rng=rng), rand(b, hkv, s, d, rng=rng), rand(b, hkv, s, d, rng=rng)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o_ref, _ = oracle.attention_ref(q, k, v, scale, mask, score)
    g = hq // hkv
    add = np.zeros((b, hq, s, s))
    for bi in range(b):
        for h in range(hq):
            vis = oracle.visible(mask, bi, np.arange(s), np.arange(s))
            add[bi, h] = np.where(vis, oracle.bias(score, h, hq, np.arange(s), np.arange(s)), -np.inf)
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1)
    o_t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, attn_mask=torch.from_numpy(add), scale=scale)
    np.testing.assert_allclose(o_ref, o_t.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mi", range(N_MASKS))
def test_matches_torch_cpu_sdpa(mi):
    for score in ALL_SCORES:
        check_against_torch_sdpa(all_masks(24, [5, 11, 8])[mi], score, seed=mi)


# ----------------------------------------------------------------------------
# closed forms

def check_causal_row0_and_q0():
    rng = np.random.default_rng(9)
    s, d = 20, 8
    q, k, v = rand(1, 1, s, d, rng=rng), rand(1, 1, s, d, rng=rng), rand(1, 1, s, d, rng=rng)
    o, lse = oracle.attention_ref(q, k, v, 0.35, MaskSpec(MASK_CAUSAL))
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])            # row 0 returns V[0] exactly
    assert lse[0, 0, 0] == pytest.approx(float(np.float32(0.35)) * float(q[0, 0, 0] @ k[0, 0, 0]), abs=1e-14)
    o0, l0 = oracle.attention_ref(np.zeros_like(q), k, v, 0.35, MaskSpec(MASK_CAUSAL))
    i = np.arange(s)
    np.testing.assert_allclose(l0[0, 0], np.log(i + 1.0), atol=1e-14)
    np.testing.assert_allclose(o0[0, 0], np.cumsum(v[0, 0], axis=0) / (i + 1.0)[:, None], atol=1e-14)


def test_causal_closed_forms():
    check_causal_row0_and_q0()


def check_window_closed_forms():
    rng = np.random.default_rng(11)
    s, d = 30, 4
    k, v = rand(1, 1, s, d, rng=rng), rand(1, 1, s, d, rng=rng)
    z = np.zeros((1, 1, s, d))
    i = np.arange(s)
    for w in (1, 3, 7):
        _, l0 = oracle.attention_ref(z, k, v, 1.0, MaskSpec(MASK_SLIDING, window=w))
        np.testing.assert_allclose(l0[0, 0], np.log(np.minimum(i + 1.0, w)), atol=1e-14)
    q = rand(1, 1, s, d, rng=rng)
    o1, _ = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_SLIDING, window=1))
    np.testing.assert_allclose(o1, v, atol=0, rtol=0)
    oa, la = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_SLIDING, window=s))
    oc, lc = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_CAUSAL))
    np.testing.assert_allclose(oa, oc, atol=1e-15)
    np.testing.assert_allclose(la, lc, atol=1e-15)


def test_sliding_window_closed_forms():
    check_window_closed_forms()


def check_prefix_closed_forms():
    rng = np.random.default_rng(12)
    s, d = 25, 4
    q, k, v = rand(1, 1, s, d, rng=rng), rand(1, 1, s, d, rng=rng), rand(1, 1, s, d, rng=rng)
    z = np.zeros_like(q)
    i = np.arange(s)
    for p in (0, 1, 6, 13):
        _, l0 = oracle.attention_ref(z, k, v, 1.0, MaskSpec(MASK_PREFIX_LM, prefix_len=p))
        np.testing.assert_allclose(l0[0, 0], np.log(np.maximum(i + 1.0, p)), atol=1e-14)
    op, lp = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_PREFIX_LM, prefix_len=0))
    oc, lc = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_CAUSAL))
    np.testing.assert_allclose(op, oc, atol=0)
    op, lp = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_PREFIX_LM, prefix_len=s))
    on, ln_ = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_NONE))
    np.testing.assert_allclose(op, on, atol=0)
    np.testing.assert_allclose(lp, ln_, atol=0)


def test_prefix_lm_closed_forms():
    check_prefix_closed_forms()


def check_document_closed_forms():
    rng = np.random.default_rng(13)
    lengths = [4, 1, 9, 6]
    s, d = sum(lengths), 4
    q, k, v = rand(1, 1, s, d, rng=rng), rand(1, 1, s, d, rng=rng), rand(1, 1, s, d, rng=rng)
    ids = doc_ids_for(lengths)
    starts = np.repeat(np.cumsum([0] + lengths[:-1]), lengths)
    i = np.arange(s)
    _, l0 = oracle.attention_ref(np.zeros_like(q), k, v, 1.0, MaskSpec(MASK_DOCUMENT, doc_ids=ids))
    np.testing.assert_allclose(l0[0, 0], np.log(i - starts + 1.0), atol=1e-14)
    o, _ = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_DOCUMENT, doc_ids=ids))
    for st in np.cumsum([0] + lengths[:-1]):
        assert np.array_equal(o[0, 0, st], v[0, 0, st])
    os_, ls_ = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_DOCUMENT, doc_ids=np.zeros((1, s), int)))
    oc, lc = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_CAUSAL))
    np.testing.assert_allclose(os_, oc, atol=0)
    np.testing.assert_allclose(ls_, lc, atol=0)


def test_document_closed_forms():
    check_document_closed_forms()


def check_and_composition():
    # sliding window W + document + causal: row i of a document starting at
    # st sees keys max(st, i - W + 1) .. i, so with Q = 0 LSE = ln(count) and
    # O = the mean of those V rows
    rng = np.random.default_rng(17)
    lengths = [4, 1, 9, 6, 2]
    s, d, w = sum(lengths), 3, 3
    k, v = rand(1, 1, s, d, rng=rng), rand(1, 1, s, d, rng=rng)
    ids = doc_ids_for(lengths)
    starts = np.repeat(np.cumsum([0] + lengths[:-1]), lengths)
    i = np.arange(s)
    first = np.maximum(starts, i - w + 1)
    m = MaskSpec(MASK_AND, window=w, doc_ids=ids, and_kinds=(MASK_SLIDING, MASK_DOCUMENT))
    o, lse = oracle.attention_ref(np.zeros((1, 1, s, d)), k, v, 1.0, m)
    np.testing.assert_allclose(lse[0, 0], np.log(i - first + 1.0), atol=1e-14)
    for r in range(s):
        np.testing.assert_allclose(o[0, 0, r], v[0, 0, first[r]:r + 1].mean(axis=0), atol=1e-14)
    # visible-pair count by documents: sum over a document of length n of
    # min(r + 1, W), r = 0..n-1
    want = sum(sum(min(r + 1, w) for r in range(n)) for n in lengths)
    assert int(oracle.visible(m, 0, i, i).sum()) == want
    # identities of the intersection: no term is no mask; one term is that
    # mask; causal adds nothing to a window or a document (both imply it);
    # the prefix adds nothing to any mask that implies causal; a window
    # longer than every document adds nothing to the document mask; one
    # document covering everything adds nothing to the window
    doc = doc_ids_for([5, 8, 3, 7], 1)
    s2 = 23
    i2 = np.arange(s2)
    base = dict(window=4, prefix_len=6, doc_ids=doc)

    def grid(kind, kinds=()):
        return oracle.visible(MaskSpec(kind, and_kinds=kinds, **base), 0, i2, i2)
    assert np.array_equal(grid(MASK_AND, ()), grid(MASK_NONE))
    for kind in (MASK_CAUSAL, MASK_SLIDING, MASK_PREFIX_LM, MASK_DOCUMENT):
        assert np.array_equal(grid(MASK_AND, (kind,)), grid(kind))
    assert np.array_equal(grid(MASK_AND, (MASK_CAUSAL, MASK_SLIDING)), grid(MASK_SLIDING))
    assert np.array_equal(grid(MASK_AND, (MASK_CAUSAL, MASK_DOCUMENT)), grid(MASK_DOCUMENT))
    assert np.array_equal(grid(MASK_AND, (MASK_CAUSAL, MASK_PREFIX_LM)), grid(MASK_CAUSAL))
    assert np.array_equal(grid(MASK_AND, (MASK_PREFIX_LM, MASK_SLIDING)), grid(MASK_SLIDING))
    assert np.array_equal(grid(MASK_AND, (MASK_PREFIX_LM, MASK_DOCUMENT)), grid(MASK_DOCUMENT))
    wide = MaskSpec(MASK_AND, window=8, doc_ids=doc, and_kinds=(MASK_SLIDING, MASK_DOCUMENT))
    assert np.array_equal(oracle.visible(wide, 0, i2, i2),
                          oracle.visible(MaskSpec(MASK_DOCUMENT, doc_ids=doc), 0, i2, i2))
    one = MaskSpec(MASK_AND, window=4, doc_ids=np.zeros((1, s2), int), and_kinds=(MASK_SLIDING, MASK_DOCUMENT))
    assert np.array_equal(oracle.visible(one, 0, i2, i2), grid(MASK_SLIDING))
    # and the window + document intersection is neither of its terms
    both = grid(MASK_AND, (MASK_SLIDING, MASK_DOCUMENT))
    assert not np.array_equal(both, grid(MASK_SLIDING)) and not np.array_equal(both, grid(MASK_DOCUMENT))
    assert np.array_equal(both, grid(MASK_SLIDING) & grid(MASK_DOCUMENT))


def test_and_composition():
    check_and_composition()


def _geometric(r, n):
    """sum_{d<n} r^d and sum_{d<n} d r^d in closed form."""
    s0 = (1.0 - r ** n) / (1.0 - r)
    s1 = r * (1.0 - n * r ** (n - 1) + (n - 1) * r ** n) / (1.0 - r) ** 2
    return s0, s1


def check_alibi_closed_form(window=None):
    """K = 0: scores are the bias alone; with V[j] = j the output is the
    bias-weighted mean position, a truncated geometric series."""
    hq, s, d = 4, 40, 3
    k = np.zeros((1, 1, s, d))
    q = np.ones((1, hq, s, d))
    v = np.tile(np.arange(s, dtype=np.float64)[:, None], (1, d))[None, None]
    mask = MaskSpec(MASK_CAUSAL) if window is None else MaskSpec(MASK_SLIDING, window=window)
    o, lse = oracle.attention_ref(q, k, v, 1.0, mask, ScoreSpec(SCORE_ALIBI))
    for h in range(hq):
        slope = 2.0 ** (-8.0 * (h + 1) / hq)
        r = math.exp(-slope)
        for i in range(s):
            n = i + 1 if window is None else min(i + 1, window)
            s0, s1 = _geometric(r, n)
            assert lse[0, h, i] == pytest.approx(math.log(s0), abs=1e-12)
            assert o[0, h, i, 0] == pytest.approx(i - s1 / s0, abs=1e-11)


def test_alibi_closed_form_causal():
    check_alibi_closed_form()


def test_alibi_closed_form_window():
    check_alibi_closed_form(window=7)


def check_rel_pos_closed_form():
    s, d, c = 30, 2, -0.25
    k = np.zeros((1, 1, s, d))
    q = np.ones((1, 2, s, d))
    v = np.tile(np.arange(s, dtype=np.float64)[:, None], (1, d))[None, None]
    o, lse = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_CAUSAL), ScoreSpec(SCORE_REL_POS, rel_scale=c))
    r = math.exp(c)                       # bias c*(i-j) = c*dist
    for i in range(s):
        s0, s1 = _geometric(r, i + 1)
        assert lse[0, 1, i] == pytest.approx(math.log(s0), abs=1e-12)
        assert o[0, 1, i, 1] == pytest.approx(i - s1 / s0, abs=1e-11)
    # ALiBi with a uniform slope is rel-pos with c = -slope (same bias c*(i-j))
    rng = np.random.default_rng(21)
    q2, k2, v2 = rand(1, 3, s, 4, rng=rng), rand(1, 3, s, 4, rng=rng), rand(1, 3, s, 4, rng=rng)
    sl = np.full(3, 0.125)
    oa, la = oracle.attention_ref(q2, k2, v2, 0.5, MaskSpec(MASK_CAUSAL), ScoreSpec(SCORE_ALIBI, slopes=sl))
    orp, lrp = oracle.attention_ref(q2, k2, v2, 0.5, MaskSpec(MASK_CAUSAL), ScoreSpec(SCORE_REL_POS, rel_scale=-0.125))
    np.testing.assert_allclose(oa, orp, atol=1e-14)
    np.testing.assert_allclose(la, lrp, atol=1e-14)


def test_rel_pos_closed_form():
    check_rel_pos_closed_form()


def check_softcap_closed_forms():
    # [FlexAttention page] §Soft-capping, read as x -> cap * tanh(x / cap).
    # (1) Two keys whose scaled scores are cap * artanh(+-y), y = a / cap:
    # the capped scores are +-a; with a = ln(3) / 2 the weights are exactly
    # 3/4 and 1/4 and LSE = ln(e^a + e^-a) = ln(4 / sqrt 3).  Scale 0.5 and
    # D = 4, so a cap applied before the scale, or without the inner division
    # or the outer factor, lands elsewhere.
    a = math.log(3.0) / 2.0
    for cap in (0.6, 4.0):
        x = cap * math.atanh(a / cap)
        q = np.zeros((1, 1, 2, 4))
        q[0, 0, :, 0] = 1.0
        k = np.zeros((1, 1, 2, 4))
        k[0, 0, 0, 0] = 2.0 * x                    # scale 0.5 -> +x
        k[0, 0, 1, 0] = -2.0 * x                   # -> -x
        v = np.array([[[[1.0, 0.0, 2.0], [0.0, 1.0, -2.0]]]])
        o, lse = oracle.attention_ref(q, k, v, 0.5, MaskSpec(MASK_NONE), ScoreSpec(SCORE_SOFTCAP, softcap=cap))
        for i in range(2):
            np.testing.assert_allclose(o[0, 0, i], [0.75, 0.25, 1.0], atol=1e-13)
            assert lse[0, 0, i] == pytest.approx(math.log(4.0 / math.sqrt(3.0)), abs=1e-13)
    rng = np.random.default_rng(57)
    s, d = 23, 8
    q, k, v = rand(1, 2, s, d, rng=rng), rand(1, 2, s, d, rng=rng), rand(1, 2, s, d, rng=rng)
    i = np.arange(s)
    # (2) a vanishing cap squashes every score to 0: uniform weights over the
    # visible keys, O = their mean and LSE = ln(count)
    o, lse = oracle.attention_ref(q, k, v, 3.0, MaskSpec(MASK_CAUSAL), ScoreSpec(SCORE_SOFTCAP, softcap=1e-9))
    np.testing.assert_allclose(lse[0, 0], np.log(i + 1.0), atol=1e-8)
    np.testing.assert_allclose(o[0, 0], np.cumsum(v[0, 0], axis=0) / (i + 1.0)[:, None], atol=1e-8)
    # (3) a cap far above every score leaves the scores unchanged
    o1, l1 = oracle.attention_ref(q, k, v, 0.4, MaskSpec(MASK_SLIDING, window=5),
                                  ScoreSpec(SCORE_SOFTCAP, softcap=1e7))
    o0, l0 = oracle.attention_ref(q, k, v, 0.4, MaskSpec(MASK_SLIDING, window=5))
    np.testing.assert_allclose(o1, o0, atol=1e-11)
    np.testing.assert_allclose(l1, l0, atol=1e-11)
    # (4) capped scores lie in [-cap, cap] (equal only where tanh rounds to
    # +-1) and never reverse the order of the raw ones
    for sc in (5.0, 0.3):
        raw = oracle.scores_block(q[0, 0], k[0, 0], sc, MaskSpec(MASK_NONE), ScoreSpec(), 0, 0, 2, i)
        cap = oracle.scores_block(q[0, 0], k[0, 0], sc, MaskSpec(MASK_NONE),
                                  ScoreSpec(SCORE_SOFTCAP, softcap=1.5), 0, 0, 2, i)
        assert np.all(np.abs(cap) <= 1.5)
        order = np.argsort(raw, axis=1)
        assert np.all(np.diff(np.take_along_axis(cap, order, axis=1), axis=1) >= 0.0)


def test_softcap_closed_forms():
    check_softcap_closed_forms()


def check_value_special_cases():
    rng = np.random.default_rng(31)
    s, d = 21, 5
    q, k = rand(2, 2, s, d, rng=rng), rand(2, 2, s, d, rng=rng)
    row = rand(d, rng=rng)
    vconst = np.broadcast_to(row, (2, 2, s, d)).copy()
    for mask in all_masks(s, [6, 6, 9]):
        for score in ALL_MODS:
            o, _ = oracle.attention_ref(q, k, vconst, 0.3, mask, score)
            np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), atol=1e-14)
    v = rand(2, 2, s, d, rng=rng)
    for mask in all_masks(s, [6, 6, 9]):
        o, lse = oracle.attention_ref(q, k, v, 0.0, mask)
        for b in range(2):
            vis = oracle.visible(mask, b, np.arange(s), np.arange(s))
            cnt = vis.sum(axis=1)
            np.testing.assert_allclose(lse[b, 0], np.log(cnt), atol=1e-14)
            np.testing.assert_allclose(o[b, 0], (vis.astype(float) @ v[b, 0]) / cnt[:, None], atol=1e-14)


def test_constant_v_and_zero_scale():
    check_value_special_cases()


def check_invariances():
    rng = np.random.default_rng(41)
    b, hq, hkv, s, d = 1, 4, 2, 19, 6
    q, k, v = rand(b, hq, s, d, rng=rng), rand(b, hkv, s, d, rng=rng), rand(b, hkv, s, d, rng=rng)
    # permuting keys and values together leaves an unmasked result unchanged
    perm = rng.permutation(s)
    o1, l1 = oracle.attention_ref(q, k, v, 0.5)
    o2, l2 = oracle.attention_ref(q, k[:, :, perm], v[:, :, perm], 0.5)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    # a per-row constant a_i added to every score (as an extra dimension with
    # q' = a_i, k' = 1, scale 1) leaves O unchanged and shifts LSE by a_i
    a = rand(s, rng=rng)
    qx = np.concatenate([q, np.broadcast_to(a[None, None, :, None], (b, hq, s, 1))], axis=-1)
    kx = np.concatenate([k, np.ones((b, hkv, s, 1))], axis=-1)
    o3, l3 = oracle.attention_ref(qx, kx, v, 1.0, MaskSpec(MASK_CAUSAL))
    o4, l4 = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_CAUSAL))
    np.testing.assert_allclose(o3, o4, atol=1e-13)
    np.testing.assert_allclose(l3, l4 + a[None, None, :], atol=1e-13)
    # GQA equals MHA on repeated kv heads (consecutive q heads share a kv head)
    g = hq // hkv
    for mask in all_masks(s, [5, 5, 9])[:4]:
        og, lg = oracle.attention_ref(q, k, v, 0.5, mask, ScoreSpec(SCORE_ALIBI))
        om, lm = oracle.attention_ref(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.5, mask,
                                      ScoreSpec(SCORE_ALIBI))
        np.testing.assert_allclose(og, om, atol=0)
        np.testing.assert_allclose(lg, lm, atol=0)


def test_invariances():
    check_invariances()


def test_fully_masked_row():
    q, k, v = rand(1, 1, 4, 3), rand(1, 1, 4, 3), rand(1, 1, 4, 3)
    o, lse = oracle.attention_ref(q, k, v, 1.0, MaskSpec(MASK_SLIDING, window=0))
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
    o, lse = oracle.attention_bruteforce(q, k, v, 1.0, MaskSpec(MASK_SLIDING, window=0))
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def test_scale_is_taken_in_float32():
    # the library receives the scale as a float32; the oracle uses that value
    q, k, v = rand(1, 1, 3, 2), rand(1, 1, 3, 2), rand(1, 1, 3, 2)
    s64 = 0.1
    _, l1 = oracle.attention_ref(q, k, v, s64)
    _, l2 = oracle.attention_ref(q, k, v, float(np.float32(s64)))
    assert np.array_equal(l1, l2)
