"""GPU parity of attn_fwd against the CPU float64 oracle, through the C ABI.

Small shapes (oracle in seconds) span several 128-row query tiles and 64-key
tiles with ragged tails, every mask kind and score modifier, both head dims,
GQA, rectangular Sq != Skv, and the BlockMask-driven path.  Full-size
workloads are checked on sampled rows the oracle computes one by one, in the
same launch configuration the bench times.
"""

import math

import numpy as np
import pytest
import torch

import attention_fa2_fwd_amd as af
import oracle
import workloads
from gpu_util import announce, compare, f64, has_document, mask_spec, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

MASKS = ["none", "causal", "sliding", "prefix_lm", "document"]
SCORES = ["none", "alibi", "rel_pos", "softcap"]


def oracle_specs(mask, score, window=0, prefix_len=0, doc_ids=None, rel_scale=1.0, softcap=0.0):
    ms = mask_spec(mask, window, prefix_len, doc_ids)
    ss = oracle.ScoreSpec(workloads.SCORE_NAMES[score], rel_scale=rel_scale, softcap=softcap)
    return ms, ss


def run_case(B, Hq, Hkv, Sq, Skv, D, dtype, mask, score, seed=0, window=100, prefix_len=70,
             doc_lengths=(50, 130, 7, 113), rel_scale=-0.05, block_mask=False, softcap=1.5,
             scale=None, mha_equal=False):
    label = (f"B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Skv{Skv} D{D} {dtype} {mask} {score} bm={block_mask}"
             f" scale={scale} softcap={softcap if score == 'softcap' else '-'}")
    q, k, v = workloads.randn_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed)
    doc_ids = None
    if has_document(mask):
        lens = list(doc_lengths)
        lens[-1] += Sq - sum(lens)
        doc_ids = torch.from_numpy(workloads.doc_ids_from_lengths(lens, B))
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    dd = doc_ids.to(dev) if doc_ids is not None else None
    bm = None
    if block_mask:
        bm = af.attn_build_block_mask(mask, B, Sq, Skv, window=window, prefix_len=prefix_len,
                                      doc_ids=dd, device=dev)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    announce(label)
    kw = dict(scale=scale, mask=mask, window=window, prefix_len=prefix_len, doc_ids=dd,
              score=score, rel_scale=rel_scale, softcap=softcap, block_mask=bm)
    out, lse = af.attn_fwd(qd, kd, vd, **kw)
    if mha_equal:
        # The same launch with every query head given its own copy of its kv
        # head: grouped heads (the four-head workgroups included) must give
        # the multi-head result bit for bit.
        g = Hq // Hkv
        o_m, l_m = af.attn_fwd(qd, kd.repeat_interleave(g, dim=1).contiguous(),
                               vd.repeat_interleave(g, dim=1).contiguous(), **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, o_m) and torch.equal(lse, l_m), label + " grouped != multi-head"
    out32 = None
    if q.dtype == torch.bfloat16:
        out32, lse32 = af.attn_fwd(qd, kd, vd, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    ms, ss = oracle_specs(mask, score, window, prefix_len, doc_ids, rel_scale, softcap)
    o_ref, l_ref = oracle.attention_ref(f64(q), f64(k), f64(v), scale, ms, ss)
    if out32 is not None:
        # the computed values (fp32 output) at the tolerance; the bf16 output
        # is exactly their rounding to nearest even
        compare(out32, lse32, o_ref, l_ref, q.dtype, label + " fp32-out")
        check_rounding(out, out32, lse, lse32)
        compare(out, lse, o_ref, l_ref, q.dtype, label + " bf16-out", out_rounding=True)
    else:
        compare(out, lse, o_ref, l_ref, q.dtype, label)
    return out, lse


def check_rounding(out_bf16, out_f32, lse_a, lse_b):
    """The bf16 output is exactly the fp32 output rounded to nearest even."""
    assert out_f32.dtype == torch.float32 and out_bf16.dtype == torch.bfloat16
    assert torch.equal(out_f32.to(torch.bfloat16), out_bf16)
    assert torch.equal(lse_a, lse_b)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("score", SCORES)
def test_bf16_small(D, mask, score):
    run_case(2, 4, 2, 300, 300, D, "bf16", mask, score, seed=D + len(mask) + len(score))


@pytest.mark.parametrize("Sq,Skv", [(200, 333), (333, 200), (64, 1000), (1, 77)])
@pytest.mark.parametrize("mask", ["none", "causal", "sliding", "prefix_lm"])
def test_bf16_rectangular(Sq, Skv, mask):
    run_case(1, 2, 1, Sq, Skv, 128, "bf16", mask, "alibi", seed=Sq + Skv)


# Unmasked D=64 runs on 128-key tiles, so its ragged ends and short key
# ranges get shapes of their own (the tile's last key past Skv, Skv < 128,
# Skv a multiple of 128, one query).
@pytest.mark.parametrize("Sq,Skv", [(200, 333), (333, 200), (64, 1000), (1, 77), (129, 256), (300, 127)])
@pytest.mark.parametrize("score", ["none", "alibi", "softcap"])
def test_bf16_rectangular_unmasked_d64(Sq, Skv, score):
    run_case(2, 4, 2, Sq, Skv, 64, "bf16", "none", score, seed=Sq + 3 * Skv)


@pytest.mark.parametrize("D", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("mask", MASKS)
def test_f32_small(D, mask):
    score = {64: "alibi", 32: "softcap", 128: "softcap"}.get(D, "none")
    run_case(1, 4, 2, 150, 150, D, "f32", mask, score, seed=D, doc_lengths=(40, 33, 77))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("softcap", [0.3, 4.0, 12.0])
def test_softcap_large_scores(D, softcap):
    # scale 1: scores of spread sqrt(D) (8 or 11), far past the small caps
    # (every score saturates towards +-cap) and bent by cap 12.  A cap far
    # above the scores is left out here: at scale 1 the softmax then rests on
    # one or two keys, and the bf16 rounding of P alone reaches the bound.
    run_case(1, 4, 2, 200, 260, D, "bf16", "causal", "softcap", seed=int(softcap * 10) + D,
             softcap=softcap, scale=1.0)


# Intersections of masks: window + document is the one that needs its own
# kernel variant; the others reduce to a single kind before launch.
AND_MASKS = ["sliding&document", "sliding&document&causal", "causal&prefix_lm", "prefix_lm&sliding",
             "document&prefix_lm&causal", "causal&sliding"]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", AND_MASKS)
@pytest.mark.parametrize("score", ["none", "alibi", "softcap"])
def test_bf16_and_masks(D, mask, score):
    run_case(2, 4, 2, 300, 300, D, "bf16", mask, score, seed=D + len(mask) + len(score), window=37)


@pytest.mark.parametrize("window", [1, 16, 64, 65, 127, 128, 129, 200, 1000])
@pytest.mark.parametrize("block_mask", [False, True])
def test_bf16_document_window_sizes(window, block_mask):
    run_case(1, 4, 4, 700, 700, 128, "bf16", "sliding&document&causal", "none", seed=window,
             window=window, doc_lengths=(300, 41, 129, 1, 229), block_mask=block_mask)


@pytest.mark.parametrize("mask", AND_MASKS)
def test_f32_and_masks(mask):
    run_case(1, 4, 2, 150, 150, 64, "f32", mask, "alibi", seed=len(mask), window=21,
             doc_lengths=(40, 33, 77))


def test_tiny_causal_f32_workload():
    w = workloads.TINY_CAUSAL_F32
    run_case(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, w.dtype, w.mask, w.score, seed=w.seed)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "sliding", "prefix_lm", "document", "sliding&document&causal"])
def test_block_mask_path_equals_dense_path(D, mask):
    """The BlockMask-driven kernel matches the oracle and, bit for bit, the
    analytic-range kernel (the same tiles hold the same visible keys).  At
    D=64 without a mask a 128-key block is one tile."""
    out_bm, lse_bm = run_case(1, 4, 4, 700, 700, D, "bf16", mask, "none", seed=5,
                              window=200, prefix_len=150, doc_lengths=(300, 41, 129, 230),
                              block_mask=True)
    out_d, lse_d = run_case(1, 4, 4, 700, 700, D, "bf16", mask, "none", seed=5,
                            window=200, prefix_len=150, doc_lengths=(300, 41, 129, 230))
    assert torch.equal(out_bm, out_d)
    assert torch.equal(lse_bm, lse_d)


# Groups of four or more query heads per kv head run as workgroups of 32
# positions of four heads each (no BlockMask): ragged position tiles (300 =
# 9 * 32 + 12), one query, rectangular shapes, groups of 4 and 8, a head
# count whose units do not fill the 8 XCDs evenly (12 heads), every mask kind
# and score form.
GQA_PACK_MASKS = ["none", "causal", "sliding", "prefix_lm", "document", "sliding&document&causal"]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", GQA_PACK_MASKS)
@pytest.mark.parametrize("score", ["none", "alibi", "softcap"])
def test_bf16_gqa_four_head_workgroups(D, mask, score):
    run_case(1, 8, 2, 300, 300, D, "bf16", mask, score, seed=D + 7 * len(mask) + len(score),
             window=77, mha_equal=True)


@pytest.mark.parametrize("Hq,Hkv,Sq,Skv", [(8, 1, 200, 333), (12, 3, 333, 200), (16, 4, 1, 77),
                                           (8, 2, 64, 1000), (12, 3, 130, 130)])
@pytest.mark.parametrize("mask", ["none", "causal", "sliding"])
def test_bf16_gqa_four_head_workgroups_shapes(Hq, Hkv, Sq, Skv, mask):
    run_case(2, Hq, Hkv, Sq, Skv, 128, "bf16", mask, "alibi", seed=Sq + Skv + Hq, window=150,
             mha_equal=True)


def test_deterministic_and_gqa_equals_mha():
    dev = torch.device("cuda")
    q, k, v = workloads.randn_qkv(1, 8, 2, 513, 513, 128, "bf16", 11)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    announce("determinism / GQA")
    o1, l1 = af.attn_fwd(q, k, v, mask="sliding", window=129, score="alibi")
    o2, l2 = af.attn_fwd(q, k, v, mask="sliding", window=129, score="alibi")
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o3, l3 = af.attn_fwd(q, kr, vr, mask="sliding", window=129, score="alibi")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_fully_masked_rows_give_zero_and_neg_inf():
    dev = torch.device("cuda")
    q, k, v = workloads.randn_qkv(1, 2, 2, 130, 130, 64, "bf16", 3)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    announce("fully masked rows")
    # prefix_lm with Skv < Sq: rows see keys j <= i or j < P; with raw indices
    # and Skv = 130 every row sees something, so use a document mask whose
    # ids never repeat at an earlier position instead: row i sees only itself.
    ids = torch.arange(130, dtype=torch.int32, device=dev)[None, :]
    out, lse = af.attn_fwd(q, k, v, mask="document", doc_ids=ids)
    torch.cuda.synchronize()
    assert torch.equal(out.float(), v.float().expand_as(out))   # one visible key: O = V row
    # explicit block mask listing nothing: every row fully masked
    bm = af.attn_build_block_mask("causal", 1, 130, 130, device=dev)
    bm.kv_num_blocks.zero_()
    out2, lse2 = af.attn_fwd(q, k, v, mask="causal", block_mask=bm)
    torch.cuda.synchronize()
    assert torch.all(out2 == 0)
    assert torch.all(torch.isneginf(lse2))


def test_explicit_alibi_slopes():
    dev = torch.device("cuda")
    q, k, v = workloads.randn_qkv(1, 4, 4, 200, 200, 64, "bf16", 9)
    slopes = torch.tensor([0.5, 0.25, 0.01, 0.0], dtype=torch.float32)
    announce("explicit alibi slopes")
    out, lse = af.attn_fwd(q.to(dev), k.to(dev), v.to(dev), mask="causal", score="alibi",
                           alibi_slopes=slopes.to(dev))
    torch.cuda.synchronize()
    ss = oracle.ScoreSpec(oracle.SCORE_ALIBI, slopes=slopes.numpy())
    o_ref, l_ref = oracle.attention_ref(f64(q), f64(k), f64(v), 1.0 / 8.0,
                                        oracle.MaskSpec(oracle.MASK_CAUSAL), ss)
    compare(out, lse, o_ref, l_ref, torch.bfloat16, "explicit slopes", out_rounding=True)


# ---------------------------------------------------------------------------
# Full-size workloads, sampled rows

def sample_rows(S, rng, extra=24):
    base = [0, 1, 63, 64, 127, 128, 129, 1023, 1024, 1025, S // 2, S - 129, S - 128, S - 65,
            S - 64, S - 2, S - 1]
    rows = set(r for r in base if 0 <= r < S)
    rows.update(int(x) for x in rng.integers(0, S, extra))
    return np.array(sorted(rows))


FULL = [workloads.DENSE_BF16, workloads.CAUSAL_BF16, workloads.GQA_WINDOW_ALIBI,
        workloads.DOCUMENT_BLOCKMASK, workloads.CAUSAL_SOFTCAP, workloads.DOC_WINDOW_BLOCKMASK]


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_full_size_sampled(w):
    dev = torch.device("cuda")
    inp = workloads.prefill_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    doc = inp["doc_ids"]
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    dd = doc.to(dev) if doc is not None else None
    bm = None
    if w.block_mask:
        bm = af.attn_build_block_mask(w.mask, w.B, w.Sq, w.Skv, window=w.window,
                                      prefix_len=w.prefix_len, doc_ids=dd, device=dev)
    announce(w.name)
    kw = dict(scale=1.0 / math.sqrt(w.D), mask=w.mask, window=w.window, prefix_len=w.prefix_len,
              doc_ids=dd, score=w.score, softcap=w.softcap, block_mask=bm)
    out, lse = af.attn_fwd(qd, kd, vd, **kw)
    out32, lse32 = af.attn_fwd(qd, kd, vd, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    # every output: the bf16 result is the fp32 result rounded to nearest even
    check_rounding(out, out32, lse, lse32)
    assert torch.isfinite(out32).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(123)
    rows = sample_rows(w.Sq, rng)
    heads = sorted({0, w.Hq - 1, w.Hq // 2 + 1})
    batches = sorted({0, w.B - 1})
    ms, ss = oracle_specs(w.mask, w.score, w.window, w.prefix_len, doc, softcap=w.softcap)
    o_ref, l_ref = oracle.attention_ref(f64(q), f64(k), f64(v), 1.0 / math.sqrt(w.D), ms, ss,
                                        rows=rows, heads=heads, batches=batches)
    sel = np.ix_(batches, heads, rows)
    compare(f64(out32)[sel], f64(lse32)[sel], o_ref, l_ref, q.dtype, w.name + " fp32-out")
    compare(f64(out)[sel], f64(lse)[sel], o_ref, l_ref, q.dtype, w.name + " bf16-out",
            out_rounding=True)
    if w.score in ("none", "softcap"):
        # Without a bias no output row concentrates on one or two keys except
        # the first rows of causal-type masks, so |O| < 4 and the bf16 output
        # also meets the bound; those first rows are checked for every head.
        compare(f64(out)[sel], f64(lse)[sel], o_ref, l_ref, q.dtype, w.name + " bf16-out")
        if w.mask != "none":
            first = np.arange(64)
            o_r, l_r = oracle.attention_ref(f64(q), f64(k), f64(v), 1.0 / math.sqrt(w.D), ms, ss,
                                            rows=first)
            compare(f64(out)[:, :, first], f64(lse)[:, :, first], o_r, l_r, q.dtype,
                    w.name + " bf16-out first rows")


def _two_batch_doc_ids(S):
    """[2, S] document ids with a different layout in each batch row, so the
    per-batch BlockMask rows (and their work order) differ."""
    rows = []
    for lens in ((100, 700, 37, S - 837), (600, 50, S - 650)):
        rows.append(np.repeat(np.arange(len(lens), dtype=np.int32), lens))
    return np.stack(rows).astype(np.int32)


@pytest.mark.parametrize("mask", ["document", "sliding&document"])
def test_block_mask_work_order_per_batch_rows(mask):
    """BlockMask launches take query tiles in order of listed work, ranked per
    batch row: with two different document layouts the result equals the
    oracle and, bit for bit, the closed-form path."""
    B, Hq, Hkv, S, D = 2, 4, 2, 1000, 128
    q, k, v = workloads.randn_qkv(B, Hq, Hkv, S, S, D, "bf16", 31)
    ids = _two_batch_doc_ids(S)
    dev = torch.device("cuda")
    qd, kd, vd, dd = q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(ids).to(dev)
    label = f"work order per batch row {mask}"
    announce(label)
    bm = af.attn_build_block_mask(mask, B, S, S, window=300, doc_ids=dd, device=dev)
    kw = dict(mask=mask, window=300, doc_ids=dd, score="alibi")
    out_bm, lse_bm = af.attn_fwd(qd, kd, vd, block_mask=bm, **kw)
    out_cf, lse_cf = af.attn_fwd(qd, kd, vd, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_bm, out_cf) and torch.equal(lse_bm, lse_cf)
    o_ref, l_ref = oracle.attention_ref(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D),
                                        mask_spec(mask, 300, doc_ids=ids),
                                        oracle.ScoreSpec(oracle.SCORE_ALIBI))
    compare(out_bm, lse_bm, o_ref, l_ref, q.dtype, label, out_rounding=True)


@pytest.mark.parametrize("S", [32768, 33024])
def test_block_mask_work_order_limit(S):
    """Up to 256 query tiles the BlockMask launch ranks them by work; past
    that it keeps the dispatch order.  Both equal the closed-form path bit
    for bit (one head, causal, D=64)."""
    q, k, v = workloads.randn_qkv(1, 1, 1, S, S, 64, "bf16", 41)
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    announce(f"work order limit S={S}")
    bm = af.attn_build_block_mask("causal", 1, S, S, device=dev)
    out_bm, lse_bm = af.attn_fwd(qd, kd, vd, mask="causal", block_mask=bm)
    out_cf, lse_cf = af.attn_fwd(qd, kd, vd, mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(out_bm, out_cf) and torch.equal(lse_bm, lse_cf)
    # a few rows against the oracle (row i sees keys 0..i)
    rows = [0, 1, 127, 128, S // 2, S - 1]
    qs = f64(q)[0, 0, rows]
    kk, vv = f64(k)[0, 0], f64(v)[0, 0]
    for n, i in enumerate(rows):
        s = (kk[: i + 1] @ qs[n]) / math.sqrt(64)
        m = s.max()
        p = np.exp(s - m)
        o = (p @ vv[: i + 1]) / p.sum()
        assert np.max(np.abs(out_bm[0, 0, i].float().cpu().numpy() - o)) <= 1e-2
        assert abs(float(lse_bm[0, 0, i]) - (m + math.log(p.sum()))) <= 1e-3
