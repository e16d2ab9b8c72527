"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a plausible wrong version (a flipped
sign, an off-by-one, a dropped term, a wrong head map, a transposed operand)
and runs the pin checks of test_oracle_pins / test_oracle_blockmask_decode
against it; at least one check must fail.  Runs on the CPU only.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as att
from oracle import block_mask as bm
from oracle import paged_decode as pdm
import test_oracle_pins as pins
import test_oracle_blockmask_decode as bpins


def _all_pins():
    pins.check_softmax_forms()
    for mi, mask in enumerate(pins.all_masks(16)):
        for si, score in enumerate(pins.ALL_MODS):
            pins.check_bruteforce(mask, score, seed=mi * 3 + si)
    pins.check_causal_row0_and_q0()
    pins.check_window_closed_forms()
    pins.check_prefix_closed_forms()
    pins.check_document_closed_forms()
    pins.check_and_composition()
    pins.check_alibi_closed_form()
    pins.check_alibi_closed_form(window=7)
    pins.check_rel_pos_closed_form()
    pins.check_softcap_closed_forms()
    pins.check_value_special_cases()
    pins.check_invariances()
    for mi in range(pins.N_MASKS):
        pins.check_against_torch_sdpa(pins.all_masks(24, [5, 11, 8])[mi], pins.ALL_SCORES[1], seed=mi)


def _wrong_bias_sign(score, hq, hq_count, i, j):
    b = _orig_bias(score, hq, hq_count, i, j)
    return -b if score.kind == att.SCORE_ALIBI else b


def _causal_exclusive(mask, b, i, j):
    v = _orig_visible(mask, b, i, j)
    if mask.kind == att.MASK_CAUSAL:
        ii = np.asarray(i)[:, None]
        jj = np.asarray(j)[None, :]
        return jj < ii
    return v


def _window_off_by_one(mask, b, i, j):
    if mask.kind == att.MASK_SLIDING:
        d = np.asarray(i)[:, None] - np.asarray(j)[None, :]
        return (d >= 0) & (d <= mask.window)
    return _orig_visible(mask, b, i, j)


def _prefix_inclusive(mask, b, i, j):
    if mask.kind == att.MASK_PREFIX_LM:
        ii = np.asarray(i)[:, None]
        jj = np.asarray(j)[None, :]
        return (jj <= ii) | (jj <= mask.prefix_len)
    return _orig_visible(mask, b, i, j)


def _document_not_causal(mask, b, i, j):
    if mask.kind == att.MASK_DOCUMENT:
        doc = np.asarray(mask.doc_ids)[b]
        return doc[np.asarray(i)][:, None] == doc[np.asarray(j)][None, :]
    return _orig_visible(mask, b, i, j)


def _softcap_no_inner_division(score, s, hq, hq_count, i, j):
    if score.kind == att.SCORE_SOFTCAP:
        return score.softcap * np.tanh(s)
    return _orig_score_mod(score, s, hq, hq_count, i, j)


def _softcap_no_outer_factor(score, s, hq, hq_count, i, j):
    if score.kind == att.SCORE_SOFTCAP:
        return np.tanh(s / score.softcap)
    return _orig_score_mod(score, s, hq, hq_count, i, j)


def _softcap_clip(score, s, hq, hq_count, i, j):
    # a hard clip instead of the smooth cap
    if score.kind == att.SCORE_SOFTCAP:
        return np.clip(s, -score.softcap, score.softcap)
    return _orig_score_mod(score, s, hq, hq_count, i, j)


def _and_as_or(mask, b, i, j):
    if mask.kind == att.MASK_AND:
        out = np.zeros((len(np.asarray(i)), len(np.asarray(j))), dtype=bool)
        for part in mask.and_kinds:
            out |= _orig_visible(att.replace(mask, kind=part, and_kinds=()), b, i, j)
        return out
    return _orig_visible(mask, b, i, j)


def _and_drops_last_term(mask, b, i, j):
    if mask.kind == att.MASK_AND and len(mask.and_kinds) > 1:
        return _orig_visible(att.replace(mask, and_kinds=mask.and_kinds[:-1]), b, i, j)
    return _orig_visible(mask, b, i, j)


def _wrong_head_map(hq, hq_count, hkv_count):
    return hq % hkv_count


def _no_scale(scale):
    return 1.0


def _no_max_shift(s):
    e = np.exp(s)
    l = e.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        return e / l[..., None], np.zeros(s.shape[:-1]), l


def _transposed_scores(q_rows, k, scale, mask, score, b, hq, hq_count, row_idx, col_idx=None):
    s = _orig_scores(q_rows, k, scale, mask, score, b, hq, hq_count, row_idx, col_idx)
    return s.T if s.shape[0] == s.shape[1] else s


_orig_bias = att.bias
_orig_score_mod = att.score_mod
_orig_visible = att.visible
_orig_scores = att.scores_block

MUTATIONS = {
    "alibi_sign": ("bias", _wrong_bias_sign),
    "causal_exclusive": ("visible", _causal_exclusive),
    "window_off_by_one": ("visible", _window_off_by_one),
    "prefix_inclusive": ("visible", _prefix_inclusive),
    "document_not_causal": ("visible", _document_not_causal),
    "gqa_head_map": ("kv_head", _wrong_head_map),
    "dropped_scale": ("_fp32_scale", _no_scale),
    "no_max_shift": ("softmax_safe3", _no_max_shift),
    "transposed_scores": ("scores_block", _transposed_scores),
    "softcap_no_inner_division": ("score_mod", _softcap_no_inner_division),
    "softcap_no_outer_factor": ("score_mod", _softcap_no_outer_factor),
    "softcap_hard_clip": ("score_mod", _softcap_clip),
    "and_as_or": ("visible", _and_as_or),
    "and_drops_last_term": ("visible", _and_drops_last_term),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    _all_pins()                                   # clean oracle passes
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(att, attr, fn)
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            _all_pins()


def _full_any(mask, batch, sq, skv, q_block=128, kv_block=128):
    num, idx, full = _orig_block_mask(mask, batch, sq, skv, q_block, kv_block)
    full = (idx >= 0).astype(np.uint8)            # "full" taken as "listed"
    return num, idx, full


_orig_block_mask = bm.block_mask_ref


def test_planted_block_mask_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "block_mask_ref", _full_any)
    with pytest.raises(AssertionError):
        for ci in range(len(bpins.CASES)):
            bpins.test_block_mask_matches_scalar_scan(ci)


def test_planted_combine_mistake_is_caught(monkeypatch):
    def bad_combine(o_parts, lse_parts):
        return np.mean(np.asarray(o_parts), axis=0), float(np.max(lse_parts))
    monkeypatch.setattr(oracle, "lse_combine_ref", bad_combine)
    with pytest.raises(AssertionError):
        bpins.test_split_combine_equals_unsplit()


def test_planted_page_gather_mistake_is_caught(monkeypatch):
    def bad_gather(k_cache, v_cache, page_table, seq_len, s):
        kk, vv = _orig_gather(k_cache, v_cache, page_table, seq_len, s)
        return kk[:, ::-1], vv                   # keys read in the wrong order
    monkeypatch.setattr(pdm, "gather_paged_kv", bad_gather)
    with pytest.raises(AssertionError):
        bpins.test_paged_decode_equals_contiguous_attention(oracle.ScoreSpec(oracle.SCORE_ALIBI))


_orig_gather = pdm.gather_paged_kv
