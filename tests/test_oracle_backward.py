"""Pins of the oracle's backward pass (oracle/backward.py).

The backward is the gradient of the forward (FlexAttention page, intro: the
backward comes from automatic differentiation), so it is pinned against
things other than its own chain rule:
* central finite differences of the oracle's forward, element by element,
  for every mask kind and score modifier on tiny shapes;
* torch's CPU autograd through scaled_dot_product_attention in float64 (a
  library routine; additive modifiers become an additive float mask);
* invariants: the gradient of a shift of every key by one vector is zero
  (the softmax is shift-invariant per row) for additive modifiers; the keys'
  dV sum to the rows' dO where every row sees a key; dO = 0 gives zeros.
Planted mistakes (the row term D dropped, the soft cap's derivative
dropped, the scale dropped from dK) must fail these pins.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bwd
from oracle import (MaskSpec, ScoreSpec, MASK_NONE, MASK_CAUSAL, MASK_SLIDING, MASK_PREFIX_LM,
                    MASK_DOCUMENT, MASK_AND, SCORE_NONE, SCORE_ALIBI, SCORE_REL_POS, SCORE_SOFTCAP)


def _ids(lengths, batch=1):
    return np.tile(np.repeat(np.arange(len(lengths)), lengths)[None, :], (batch, 1))


S_TINY = 9
MASKS = [
    MaskSpec(MASK_NONE),
    MaskSpec(MASK_CAUSAL),
    MaskSpec(MASK_SLIDING, window=3),
    MaskSpec(MASK_PREFIX_LM, prefix_len=4),
    MaskSpec(MASK_DOCUMENT, doc_ids=_ids([3, 2, 4])),
    MaskSpec(MASK_AND, window=2, doc_ids=_ids([3, 2, 4]), and_kinds=(MASK_SLIDING, MASK_DOCUMENT)),
]
SCORES = [ScoreSpec(SCORE_NONE), ScoreSpec(SCORE_ALIBI), ScoreSpec(SCORE_REL_POS, rel_scale=-0.3),
          ScoreSpec(SCORE_SOFTCAP, softcap=0.8)]


def _inputs(seed, b=1, hq=2, hkv=1, s=S_TINY, d=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, hq, s, d))
    k = rng.standard_normal((b, hkv, s, d))
    v = rng.standard_normal((b, hkv, s, d))
    do = rng.standard_normal((b, hq, s, d))
    return q, k, v, do


def _loss(q, k, v, do, scale, mask, score):
    o, _ = oracle.attention_ref(q, k, v, scale, mask, score)
    return float(np.sum(o * do))


def check_finite_differences(mask, score, seed=0, h=1e-5):
    q, k, v, do = _inputs(seed)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward_ref(q, k, v, do, scale, mask, score)
    for name, t, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            old = t[idx]
            t[idx] = old + h
            lp = _loss(q, k, v, do, scale, mask, score)
            t[idx] = old - h
            lm = _loss(q, k, v, do, scale, mask, score)
            t[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8, err_msg=f"d{name}")


@pytest.mark.parametrize("mi", range(len(MASKS)))
@pytest.mark.parametrize("si", range(len(SCORES)))
def test_backward_matches_finite_differences(mi, si):
    check_finite_differences(MASKS[mi], SCORES[si], seed=7 * mi + si)


def check_against_torch_autograd(mask, score, seed=0):
    rng = np.random.default_rng(seed)
    b, hq, hkv, s, d = 2, 4, 2, 24, 8
    q, k, v, do = (rng.standard_normal(sh) for sh in ((b, hq, s, d), (b, hkv, s, d), (b, hkv, s, d),
                                                       (b, hq, s, d)))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    dq, dk, dv = oracle.attention_backward_ref(q, k, v, do, scale, mask, score)
    g = hq // hkv
    add = np.zeros((b, hq, s, s))
    for bi in range(b):
        for h in range(hq):
            vis = oracle.visible(mask, bi, np.arange(s), np.arange(s))
            add[bi, h] = np.where(vis, oracle.bias(score, h, hq, np.arange(s), np.arange(s)), -np.inf)
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(g, dim=1), vt.repeat_interleave(g, dim=1),
        attn_mask=torch.from_numpy(add), scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mi", [0, 1, 2, 3])
@pytest.mark.parametrize("si", [0, 1, 2])
def test_backward_matches_torch_autograd(mi, si):
    # masks whose every row sees a key (the library returns NaN for a row
    # with none); the document masks are covered by the finite differences
    check_against_torch_autograd(MASKS[mi], SCORES[si], seed=3 * mi + si)


def check_invariants():
    rng = np.random.default_rng(5)
    b, hq, hkv, s, d = 1, 4, 2, 17, 5
    q, k, v, do = (rng.standard_normal(sh) for sh in ((b, hq, s, d), (b, hkv, s, d), (b, hkv, s, d),
                                                       (b, hq, s, d)))
    for mask in MASKS[:4] + [MaskSpec(MASK_DOCUMENT, doc_ids=_ids([5, 1, 11]))]:
        for score in SCORES[:3]:
            dq, dk, dv = oracle.attention_backward_ref(q, k, v, do, 0.6, mask, score)
            # shifting every key of a head by one vector c adds q_i . c to all
            # of row i's scores: no change, so the keys' dK sum to zero
            np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
            # P's rows sum to one, so the keys' dV sum to the rows' dO
            g = hq // hkv
            want = do.reshape(b, hkv, g, s, d).sum(axis=(2, 3))
            np.testing.assert_allclose(dv.sum(axis=2), want, atol=1e-12)
    z = oracle.attention_backward_ref(q, k, v, np.zeros_like(do), 0.6, MASKS[1], SCORES[1])
    assert all(np.all(t == 0.0) for t in z)
    # the soft cap breaks the shift invariance: its dK do not sum to zero
    _, dk, _ = oracle.attention_backward_ref(q, k, v, do, 0.6, MASKS[0], SCORES[3])
    assert np.abs(dk.sum(axis=2)).max() > 1e-3


def test_backward_invariants():
    check_invariants()


def test_softmax_row_dot():
    rng = np.random.default_rng(2)
    o, do = rng.standard_normal((2, 3, 5, 4)), rng.standard_normal((2, 3, 5, 4))
    d = oracle.softmax_row_dot_ref(o, do)
    assert d.shape == (2, 3, 5)
    assert d[1, 2, 3] == pytest.approx(float(o[1, 2, 3] @ do[1, 2, 3]), abs=1e-15)


def test_fully_masked_rows_have_zero_gradients():
    q, k, v, do = _inputs(3)
    dq, dk, dv = oracle.attention_backward_ref(q, k, v, do, 1.0, MaskSpec(MASK_SLIDING, window=0))
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0)


# ---------------------------------------------------------------------------
# planted mistakes

def _all_pins():
    for mi in range(len(MASKS)):
        for si in range(len(SCORES)):
            check_finite_differences(MASKS[mi], SCORES[si], seed=7 * mi + si)
    check_invariants()


_orig_rows = bwd.attention_backward_rows


def _no_row_term(q_rows, k, v, do_rows, row_idx, b, hq, hq_count, scale, mask=MaskSpec(), score=ScoreSpec()):
    # dS = P * dP (D dropped): recompute with dO orthogonalised away from O is
    # not what the softmax Jacobian gives
    q_rows = np.asarray(q_rows, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s_fp = float(np.float32(scale))
    s = oracle.scores_block(q_rows, k, scale, mask, score, b, hq, hq_count, row_idx)
    p, _, _ = oracle.softmax_safe3(s)
    dp = np.asarray(do_rows) @ v.T
    dx = p * dp * bwd._score_mod_grad(score, s_fp * (q_rows @ k.T))
    return s_fp * (dx @ k), s_fp * (dx.T @ q_rows), p.T @ np.asarray(do_rows)


def _dk_unscaled(*args, **kw):
    dq, dk, dv = _orig_rows(*args, **kw)
    s_fp = float(np.float32(args[8]))
    return dq, dk / s_fp, dv


@pytest.mark.parametrize("name,attr,fn", [
    ("row_term_dropped", "attention_backward_rows", _no_row_term),
    ("dk_scale_dropped", "attention_backward_rows", _dk_unscaled),
    ("softcap_derivative_dropped", "_score_mod_grad", lambda score, x: np.ones_like(x)),
])
def test_planted_backward_mistake_is_caught(name, attr, fn, monkeypatch):
    _all_pins()
    monkeypatch.setattr(bwd, attr, fn)
    with pytest.raises(AssertionError):
        _all_pins()
