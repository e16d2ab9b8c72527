"""GPU parity of attn_bwd against the CPU float64 oracle, through the C ABI.

The backward takes the forward's bf16 output O and float32 LSE from attn_fwd
on the same inputs (the way a caller uses it) and a seeded dO; the oracle
differentiates its own forward from q, k, v, dO alone.  Every gradient
element is compared, on shapes that span several 128-row query tiles,
64-key tiles and 32-query tiles with ragged tails, every mask kind and score
modifier, both head dims and GQA; the causal B=4 H=16 S=2048 D=64 shape the
bench times is checked on whole heads.

Tolerance (bf16 inputs, fp32 gradients).  Each gradient is a sum of
products in which one factor, P (for dV) or dS (for dK, dQ), is rounded to
bf16 first: relative error at most 2^-9 per term, so the sum's relative
error is at most 2^-9 when its terms share a sign and about 2^-9 / sqrt(3)
when their signs are random; the row term D, formed from the bf16 output O,
adds a like amount to dS.  Each gradient tensor G is held to
    mean |G - G_ref| <= 2^-8 * max(mean |G_ref|, FLOOR)
    max  |G - G_ref| <= 1e-2 * max(max |G_ref|, FLOOR)
(the forward's max-abs bound, relative), with FLOOR = 1/16 for tensors whose
exact value is zero (one key: P = 1, dS = 0, dQ = 0).
"""

import math

import numpy as np
import pytest
import torch

import attention_fa2_fwd_amd as af
import oracle
import workloads
from gpu_util import announce, f64, has_document, mask_spec, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

BWD_MAX_REL = 1.0e-2
BWD_MEAN_REL = 2.0 ** -8
FLOOR = 1.0 / 16

MASKS = ["none", "causal", "sliding", "prefix_lm", "document", "sliding&document&causal"]
SCORES = ["none", "alibi", "rel_pos", "softcap"]


def compare_grads(got, ref, label):
    summary = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = f64(g)
        assert g.shape == r.shape, (name, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite"
        err = np.abs(g - r)
        scale_max = max(np.abs(r).max(), FLOOR)
        scale_mean = max(np.abs(r).mean(), FLOOR)
        summary[name] = (float(err.max() / scale_max), float(err.mean() / scale_mean))
    print(f"{label}: " + ", ".join(f"{n} max/|max| {a:.2e} mean/|mean| {b:.2e}"
                                   for n, (a, b) in summary.items()), flush=True)
    for name, (a, b) in summary.items():
        assert a <= BWD_MAX_REL, f"{label} {name}: max rel {a:.3e}"
        assert b <= BWD_MEAN_REL, f"{label} {name}: mean rel {b:.3e}"


def run_bwd(B, Hq, Hkv, Sq, Skv, D, mask, score, seed=0, window=100, prefix_len=70,
            doc_lengths=(50, 130, 7, 113), softcap=1.5, scale=None, block_mask=False):
    label = f"bwd B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Skv{Skv} D{D} {mask} {score} bm={block_mask}"
    q, k, v = workloads.randn_qkv(B, Hq, Hkv, Sq, Skv, D, "bf16", seed)
    do = workloads.randn_qkv(B, Hq, Hkv, Sq, Skv, D, "bf16", seed + 1000)[0]
    doc_ids = None
    if has_document(mask):
        lens = list(doc_lengths)
        lens[-1] += Sq - sum(lens)
        doc_ids = torch.from_numpy(workloads.doc_ids_from_lengths(lens, B))
    dev = torch.device("cuda")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    dd = doc_ids.to(dev) if doc_ids is not None else None
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    kw = dict(scale=scale, mask=mask, window=window, prefix_len=prefix_len, doc_ids=dd, score=score,
              rel_scale=-0.05, softcap=softcap)
    announce(label)
    out, lse = af.attn_fwd(qd, kd, vd, **kw)
    bm = None
    if block_mask:
        bm = af.attn_block_mask_transpose(
            af.attn_build_block_mask(mask, B, Sq, Skv, window=window, prefix_len=prefix_len, doc_ids=dd,
                                     device=dev))
    dq, dk, dv = af.attn_bwd(qd, kd, vd, out, lse, dod, block_mask=bm, **kw)
    torch.cuda.synchronize()
    ms = mask_spec(mask, window, prefix_len, doc_ids)
    ss = oracle.ScoreSpec(workloads.SCORE_NAMES[score], rel_scale=-0.05, softcap=softcap)
    ref = oracle.attention_backward_ref(f64(q), f64(k), f64(v), f64(do), scale, ms, ss)
    compare_grads((dq, dk, dv), ref, label)
    return dq, dk, dv


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("score", SCORES)
def test_bwd_small(D, mask, score):
    run_bwd(2, 4, 2, 300, 300, D, mask, score, seed=D + len(mask) + len(score), window=37)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", MASKS)
def test_bwd_block_mask_path(D, mask):
    """With the BlockMask the backward matches the oracle and, bit for bit,
    the closed-form path (the extra tiles that path visits add exact zeros)."""
    kw = dict(seed=11 + D, window=150, prefix_len=200, doc_lengths=(300, 41, 129, 1, 229))
    g_bm = run_bwd(1, 4, 2, 700, 700, D, mask, "alibi", block_mask=True, **kw)
    g_cf = run_bwd(1, 4, 2, 700, 700, D, mask, "alibi", **kw)
    for a, b in zip(g_bm, g_cf):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mask", ["document", "sliding&document"])
@pytest.mark.parametrize("block_mask", [False, True])
def test_bwd_unsorted_document_ids(mask, block_mask):
    # ids drawn at random from 5 values: neither sorted nor contiguous
    B, Hq, Hkv, S, D = 1, 4, 2, 400, 64
    q, k, v = workloads.randn_qkv(B, Hq, Hkv, S, S, D, "bf16", 21)
    do = workloads.randn_qkv(B, Hq, Hkv, S, S, D, "bf16", 22)[0]
    ids = torch.from_numpy(np.random.default_rng(23).integers(0, 5, size=(B, S)).astype(np.int32))
    dev = torch.device("cuda")
    qd, kd, vd, dod, dd = q.to(dev), k.to(dev), v.to(dev), do.to(dev), ids.to(dev)
    kw = dict(mask=mask, window=90, doc_ids=dd, score="rel_pos", rel_scale=-0.05)
    label = f"bwd unsorted ids {mask} bm={block_mask}"
    announce(label)
    out, lse = af.attn_fwd(qd, kd, vd, **kw)
    bm = None
    if block_mask:
        bm = af.attn_build_block_mask(mask, B, S, S, window=90, doc_ids=dd, device=dev)
    grads = af.attn_bwd(qd, kd, vd, out, lse, dod, block_mask=bm, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_backward_ref(f64(q), f64(k), f64(v), f64(do), 1.0 / math.sqrt(D),
                                        mask_spec(mask, 90, doc_ids=ids),
                                        oracle.ScoreSpec(oracle.SCORE_REL_POS, rel_scale=-0.05))
    compare_grads(grads, ref, label)


@pytest.mark.parametrize("Sq,Skv", [(200, 333), (333, 200), (64, 1000), (1, 77), (77, 1)])
@pytest.mark.parametrize("mask", ["none", "causal", "sliding", "prefix_lm"])
def test_bwd_rectangular(Sq, Skv, mask):
    run_bwd(1, 2, 1, Sq, Skv, 128, mask, "alibi", seed=Sq + Skv)


@pytest.mark.parametrize("G", [1, 3, 8])
def test_bwd_gqa_groups(G):
    run_bwd(1, 2 * G, 2, 260, 260, 64, "causal", "none", seed=G)


# Groups of four or more query heads per kv head run the dQ pass as
# workgroups of 32 positions x 4 heads (no BlockMask): against the oracle,
# and dQ bit for bit against the same call with K/V expanded to every query
# head (dK / dV sum the group's heads, so they are held to the oracle only).
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", MASKS)
def test_bwd_gqa_four_head_dq_workgroups(D, mask):
    B, Hq, Hkv, S = 1, 8, 2, 300
    run_bwd(B, Hq, Hkv, S, S, D, mask, "alibi", seed=D + len(mask), window=77)
    q, k, v = workloads.randn_qkv(B, Hq, Hkv, S, S, D, "bf16", D + len(mask))
    do = workloads.randn_qkv(B, Hq, Hkv, S, S, D, "bf16", D + len(mask) + 1000)[0]
    dev = torch.device("cuda")
    dd = None
    if has_document(mask):
        lens = [50, 130, 7, 113]
        lens[-1] += S - sum(lens)
        dd = torch.from_numpy(workloads.doc_ids_from_lengths(lens, B)).to(dev)
    kw = dict(mask=mask, window=77, prefix_len=70, doc_ids=dd, score="alibi")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    out, lse = af.attn_fwd(qd, kd, vd, **kw)
    dq, _, _ = af.attn_bwd(qd, kd, vd, out, lse, dod, **kw)
    kr = kd.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    vr = vd.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    dq_m, _, _ = af.attn_bwd(qd, kr, vr, out, lse, dod, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq_m)


def test_bwd_deterministic():
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in workloads.randn_qkv(1, 8, 2, 700, 700, 128, "bf16", 3))
    do = workloads.randn_qkv(1, 8, 2, 700, 700, 128, "bf16", 4)[0].to(dev)
    announce("bwd deterministic")
    out, lse = af.attn_fwd(q, k, v, mask="sliding", window=300, score="alibi")
    g1 = af.attn_bwd(q, k, v, out, lse, do, mask="sliding", window=300, score="alibi")
    g2 = af.attn_bwd(q, k, v, out, lse, do, mask="sliding", window=300, score="alibi")
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bwd_rows_without_keys():
    # sliding window 50 with Sq = 300 > Skv = 100: rows 149.. see no key
    # (O = 0, LSE = -inf) and must give dQ = 0 and add nothing to dK, dV
    dq, _, _ = run_bwd(1, 2, 1, 300, 100, 64, "sliding", "alibi", seed=8, window=50)
    assert torch.all(dq[:, :, 149:] == 0)
    # no key at all: zero dQ, empty dK and dV
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in workloads.randn_qkv(1, 2, 1, 50, 0, 64, "bf16", 5))
    do = workloads.randn_qkv(1, 2, 1, 50, 0, 64, "bf16", 6)[0].to(dev)
    announce("bwd no keys")
    out, lse = af.attn_fwd(q, k, v)
    dq, dk, dv = af.attn_bwd(q, k, v, out, lse, do)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0


def test_bwd_causal_headline_shape_whole_heads():
    w = workloads.CAUSAL_BF16
    dev = torch.device("cuda")
    q, k, v = workloads.randn_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, "bf16", w.seed)
    do = workloads.randn_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, "bf16", w.seed + 1000)[0]
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    announce("bwd causal headline shape")
    out, lse = af.attn_fwd(qd, kd, vd, mask="causal")
    dq, dk, dv = af.attn_bwd(qd, kd, vd, out, lse, dod, mask="causal")
    torch.cuda.synchronize()
    for b, hq in ((0, 0), (w.B - 1, w.Hq - 1), (1, 7)):
        sl = (slice(b, b + 1), slice(hq, hq + 1))
        ref = oracle.attention_backward_ref(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]),
                                            1.0 / math.sqrt(w.D), oracle.MaskSpec(oracle.MASK_CAUSAL))
        compare_grads((dq[sl], dk[sl], dv[sl]), ref, f"bwd causal headline b{b} h{hq}")


@pytest.mark.parametrize("mask", ["causal", "none"])
def test_bwd_alibi_long_rows(mask):
    """ALiBi backward over 4096 positions without a window (B=1, Hq=4, Hkv=1,
    D=64): the kernels split bias2 (j - i) into a per-query and a per-key
    part relative to the workgroup's first key, whose magnitudes grow with
    the distance; with no causal mask the later keys carry the largest
    scores of each row."""
    run_bwd(1, 4, 1, 4096, 4096, 64, mask, "alibi", seed=31)


def test_bwd_gqa_window_alibi_headline_shape_one_kv_group():
    """The GQA window 1024 + ALiBi backward at its benchmarked shape (B=2,
    Hq=32, Hkv=8, S=8192, D=128): one whole kv group (the last batch row's kv
    head 7 and its query heads 28..31) against the oracle, dQ of the four
    heads and the group's dK, dV.  Far positions make the bias terms large,
    which the kernels split into a per-query and a per-key part."""
    w = workloads.GQA_WINDOW_ALIBI
    dev = torch.device("cuda")
    q, k, v = workloads.randn_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, "bf16", w.seed)
    do = workloads.randn_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, "bf16", w.seed + 1000)[0]
    kw = dict(mask="sliding", window=w.window, score="alibi")
    announce("bwd gqa window alibi headline shape, kv group b1 h7")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    out, lse = af.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = af.attn_bwd(qd, kd, vd, out, lse, dod, **kw)
    torch.cuda.synchronize()
    b, hkv, g = w.B - 1, w.Hkv - 1, w.Hq // w.Hkv
    hs = slice(hkv * g, hkv * g + g)
    slopes = oracle.alibi_slopes(w.Hq)[hs]
    ref = oracle.attention_backward_ref(f64(q[b:b + 1, hs]), f64(k[b:b + 1, hkv:hkv + 1]),
                                        f64(v[b:b + 1, hkv:hkv + 1]), f64(do[b:b + 1, hs]),
                                        1.0 / math.sqrt(w.D), oracle.MaskSpec(oracle.MASK_SLIDING, window=w.window),
                                        oracle.ScoreSpec(oracle.SCORE_ALIBI, slopes=slopes))
    compare_grads((dq[b:b + 1, hs], dk[b:b + 1, hkv:hkv + 1], dv[b:b + 1, hkv:hkv + 1]), ref,
                  "bwd gqa window alibi headline shape")


def test_bwd_document_block_mask_headline_shape_sampled_dq_rows():
    """The document BlockMask backward at its benchmarked shape (B=1, H=16,
    S=16384, D=128, the drawn document layout): dQ on sampled rows of two
    heads (the first and last row of the first documents, and rows spread
    over the sequence) against the oracle's rows, which need only those
    rows' scores."""
    w = workloads.DOCUMENT_BLOCKMASK
    dev = torch.device("cuda")
    inp = workloads.prefill_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    ids = inp["doc_ids"]
    do = workloads.randn_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, "bf16", w.seed + 1000)[0]
    qd, kd, vd, dod, dd = q.to(dev), k.to(dev), v.to(dev), do.to(dev), ids.to(dev)
    announce("bwd document BlockMask headline shape, sampled dq rows")
    out, lse = af.attn_fwd(qd, kd, vd, mask="document", doc_ids=dd)
    bm = af.attn_block_mask_transpose(af.attn_build_block_mask("document", w.B, w.Sq, w.Skv, doc_ids=dd,
                                                               device=dev))
    dq, _, _ = af.attn_bwd(qd, kd, vd, out, lse, dod, mask="document", doc_ids=dd, block_mask=bm)
    torch.cuda.synchronize()
    starts = np.cumsum([0] + list(inp["doc_lengths"]))
    rows = set(np.linspace(0, w.Sq - 1, 24).astype(int).tolist())
    for a_, b_ in zip(starts[:12], starts[1:13]):
        rows.update((int(a_), int(b_) - 1))
    rows = np.array(sorted(r for r in rows if r < w.Sq))
    ms = oracle.MaskSpec(oracle.MASK_DOCUMENT, doc_ids=ids.numpy())
    for hq in (0, w.Hq - 1):
        dq_ref, _, _ = oracle.attention_backward_rows(f64(q[0, hq])[rows], f64(k[0, hq]), f64(v[0, hq]),
                                                      f64(do[0, hq])[rows], rows, 0, hq, w.Hq,
                                                      1.0 / math.sqrt(w.D), ms)
        got = f64(dq[0, hq])[rows]
        err = np.abs(got - dq_ref)
        a = err.max() / max(np.abs(dq_ref).max(), FLOOR)
        m = err.mean() / max(np.abs(dq_ref).mean(), FLOOR)
        print(f"bwd document headline h{hq} {len(rows)} rows: dq max/|max| {a:.2e} mean/|mean| {m:.2e}", flush=True)
        assert a <= BWD_MAX_REL and m <= BWD_MEAN_REL, (hq, a, m)


@pytest.mark.parametrize("mask", ["document", "sliding&document"])
def test_bwd_block_mask_work_order_per_batch_rows(mask):
    """Both backward passes take BlockMask tiles in order of listed work,
    ranked per batch row: with a different document layout in each batch row
    the gradients equal the oracle's and, bit for bit, the closed-form
    path's."""
    B, Hq, Hkv, S, D = 2, 4, 2, 1000, 64
    q, k, v = workloads.randn_qkv(B, Hq, Hkv, S, S, D, "bf16", 51)
    do = workloads.randn_qkv(B, Hq, Hkv, S, S, D, "bf16", 52)[0]
    rows = []
    for lens in ((100, 700, 37, S - 837), (600, 50, S - 650)):
        rows.append(np.repeat(np.arange(len(lens), dtype=np.int32), lens))
    ids = torch.from_numpy(np.stack(rows).astype(np.int32))
    dev = torch.device("cuda")
    qd, kd, vd, dod, dd = q.to(dev), k.to(dev), v.to(dev), do.to(dev), ids.to(dev)
    kw = dict(mask=mask, window=300, doc_ids=dd, score="alibi")
    label = f"bwd work order per batch row {mask}"
    announce(label)
    out, lse = af.attn_fwd(qd, kd, vd, **kw)
    bm = af.attn_block_mask_transpose(af.attn_build_block_mask(mask, B, S, S, window=300, doc_ids=dd,
                                                               device=dev))
    g_bm = af.attn_bwd(qd, kd, vd, out, lse, dod, block_mask=bm, **kw)
    g_cf = af.attn_bwd(qd, kd, vd, out, lse, dod, **kw)
    torch.cuda.synchronize()
    for a, b in zip(g_bm, g_cf):
        assert torch.equal(a, b)
    ref = oracle.attention_backward_ref(f64(q), f64(k), f64(v), f64(do), 1.0 / math.sqrt(D),
                                        mask_spec(mask, 300, doc_ids=ids),
                                        oracle.ScoreSpec(oracle.SCORE_ALIBI))
    compare_grads(g_bm, ref, label)
