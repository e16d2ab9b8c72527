"""GPU parity of attn_build_block_mask (bit-exact against the oracle) and of
attn_paged_decode (against the oracle within the bf16 tolerances), through
the C ABI, including the full-size document and decode workloads."""

import math

import numpy as np
import pytest
import torch

import attention_fa2_fwd_amd as af
import oracle
import workloads
from gpu_util import announce, compare, f64, has_document, mask_spec, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _ids(lengths, batch=1):
    return workloads.doc_ids_from_lengths(lengths, batch)


BM_CASES = [
    ("none", 2, 300, 300, 128, 128, dict()),
    ("causal", 1, 2048, 2048, 128, 128, dict()),
    ("causal", 2, 300, 517, 64, 32, dict()),
    ("sliding", 1, 8192, 8192, 128, 128, dict(window=1024)),
    ("sliding", 1, 1000, 1000, 128, 64, dict(window=37)),
    ("prefix_lm", 1, 777, 777, 128, 128, dict(prefix_len=300)),
    ("prefix_lm", 1, 640, 640, 16, 1024, dict(prefix_len=0)),
    ("document", 2, 1000, 1000, 128, 128, dict(lengths=[300, 1, 129, 127, 443])),
    ("document", 1, 999, 999, 48, 80, dict(lengths=[10, 500, 489])),
    # ids that are neither sorted nor contiguous: every decision path of the
    # builder (summary tests, single-id blocks, the general scan)
    ("document", 2, 700, 700, 64, 64, dict(random_ids=4)),
    ("document", 1, 513, 513, 32, 128, dict(random_ids=40)),
    ("document", 1, 600, 600, 128, 128, dict(pattern=[(0, 100), (1, 50), (0, 80), (2, 200), (1, 170)])),
    ("document", 1, 257, 257, 128, 128, dict(lengths=[257])),     # one id; a 1-row last block
    # window + document (+ causal): interval test, document summary, and the
    # scan of the pairs inside a window that covers part of a block
    ("sliding&document", 2, 1000, 1000, 128, 128, dict(window=100, lengths=[300, 1, 129, 127, 443])),
    ("sliding&document&causal", 1, 999, 999, 48, 80, dict(window=37, lengths=[10, 500, 489])),
    ("sliding&document", 2, 700, 700, 64, 64, dict(window=50, random_ids=4)),
    ("sliding&document", 1, 513, 513, 32, 128, dict(window=200, random_ids=40)),
    ("sliding&document&causal", 1, 600, 600, 128, 128,
     dict(window=130, pattern=[(0, 100), (1, 50), (0, 80), (2, 200), (1, 170)])),
    ("sliding&document", 1, 4096, 4096, 128, 128, dict(window=1, lengths=[1000, 3000, 96])),
    ("sliding&document", 1, 4096, 4096, 128, 128, dict(window=5000, lengths=[1000, 3000, 96])),
    ("causal&prefix_lm&sliding", 1, 777, 777, 128, 128, dict(window=300, prefix_len=500)),
]


def _case_doc_ids(B, S, kw):
    if "lengths" in kw:
        return _ids(kw["lengths"], B)
    if "random_ids" in kw:
        rng = np.random.default_rng(7)
        return rng.integers(0, kw["random_ids"], size=(B, S)).astype(np.int32)
    row = np.concatenate([np.full(n, d, np.int32) for d, n in kw["pattern"]])
    assert row.size == S
    return np.tile(row[None, :], (B, 1))


@pytest.mark.parametrize("case", range(len(BM_CASES)))
def test_block_mask_bit_exact(case):
    mask, B, Sq, Skv, qb, kb, kw = BM_CASES[case]
    dev = torch.device("cuda")
    doc = None
    if has_document(mask):
        doc = torch.from_numpy(_case_doc_ids(B, Sq, kw))
    announce(f"block mask {BM_CASES[case][:6]}")
    bm = af.attn_build_block_mask(mask, B, Sq, Skv, q_block=qb, kv_block=kb,
                                  window=kw.get("window", 0), prefix_len=kw.get("prefix_len", 0),
                                  doc_ids=doc.to(dev) if doc is not None else None, device=dev)
    torch.cuda.synchronize()
    ms = mask_spec(mask, kw.get("window", 0), kw.get("prefix_len", 0), doc)
    num, idx, full = oracle.block_mask_ref(ms, B, Sq, Skv, qb, kb)
    assert np.array_equal(bm.kv_num_blocks.cpu().numpy(), num)
    assert np.array_equal(bm.kv_indices.cpu().numpy(), idx)
    assert np.array_equal(bm.kv_full.cpu().numpy(), full)


@pytest.mark.parametrize("case", range(len(BM_CASES)))
def test_block_mask_transpose_bit_exact(case):
    mask, B, Sq, Skv, qb, kb, kw = BM_CASES[case]
    dev = torch.device("cuda")
    doc = torch.from_numpy(_case_doc_ids(B, Sq, kw)) if has_document(mask) else None
    announce(f"block mask transpose {BM_CASES[case][:6]}")
    bm = af.attn_build_block_mask(mask, B, Sq, Skv, q_block=qb, kv_block=kb,
                                  window=kw.get("window", 0), prefix_len=kw.get("prefix_len", 0),
                                  doc_ids=doc.to(dev) if doc is not None else None, device=dev)
    bt = af.attn_block_mask_transpose(bm)
    torch.cuda.synchronize()
    ms = mask_spec(mask, kw.get("window", 0), kw.get("prefix_len", 0), doc)
    num, idx, full = oracle.block_mask_cols_ref(ms, B, Sq, Skv, qb, kb)
    assert np.array_equal(bt.q_num_blocks.cpu().numpy(), num)
    assert np.array_equal(bt.q_indices.cpu().numpy(), idx)
    assert np.array_equal(bt.q_full.cpu().numpy(), full)


def test_block_mask_document_window_workload():
    w = workloads.DOC_WINDOW_BLOCKMASK
    dev = torch.device("cuda")
    lengths = workloads.doc_lengths(w.Sq, seed=w.seed)
    doc = torch.from_numpy(_ids(lengths, w.B))
    announce("block mask document + window workload")
    bm = af.attn_build_block_mask(w.mask, w.B, w.Sq, w.Skv, window=w.window, doc_ids=doc.to(dev),
                                  device=dev)
    torch.cuda.synchronize()
    num, idx, full = oracle.block_mask_ref(mask_spec(w.mask, w.window, doc_ids=doc), w.B, w.Sq, w.Skv,
                                           128, 128)
    assert np.array_equal(bm.kv_num_blocks.cpu().numpy(), num)
    assert np.array_equal(bm.kv_indices.cpu().numpy(), idx)
    assert np.array_equal(bm.kv_full.cpu().numpy(), full)
    assert int(num.sum()) == 890 and int(full.sum()) == 594


def test_block_mask_document_workload():
    w = workloads.DOCUMENT_BLOCKMASK
    dev = torch.device("cuda")
    lengths = workloads.doc_lengths(w.Sq, seed=w.seed)
    doc = torch.from_numpy(_ids(lengths, w.B))
    announce("block mask document workload")
    bm = af.attn_build_block_mask("document", w.B, w.Sq, w.Skv, doc_ids=doc.to(dev), device=dev)
    torch.cuda.synchronize()
    num, idx, full = oracle.block_mask_ref(oracle.MaskSpec(oracle.MASK_DOCUMENT, doc_ids=doc.numpy()),
                                           w.B, w.Sq, w.Skv, 128, 128)
    assert np.array_equal(bm.kv_num_blocks.cpu().numpy(), num)
    assert np.array_equal(bm.kv_indices.cpu().numpy(), idx)
    assert np.array_equal(bm.kv_full.cpu().numpy(), full)
    assert int(num.sum()) == 1348 and int(full.sum()) == 1024


# ---------------------------------------------------------------------------
# paged decode

def small_decode_inputs(lengths, hq=8, hkv=2, max_pages=80, seed=0, poison=False):
    w = workloads.DecodeWorkload("small", len(lengths), hq, hkv, 128, max_pages=max_pages, seed=seed)
    inp = workloads.decode_inputs(w, device="cpu", lengths=np.array(lengths))
    if poison:
        # NaN in every slot no sequence owns and in the unused tail of the
        # last page of each sequence; -1 already fills unused table entries
        owned = torch.zeros(inp["k_cache"].shape[0], 16, dtype=torch.bool)
        table = inp["page_table"].numpy()
        for s, L in enumerate(lengths):
            for t in range(L):
                owned[table[s, t // 16], t % 16] = True
        kc, vc = inp["k_cache"], inp["v_cache"]
        nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
        for p in range(kc.shape[0]):
            for slot in range(16):
                if not owned[p, slot]:
                    kc[p, :, slot] = nan
                    vc[p, :, slot] = nan
    return inp


def run_decode(inp, score="none", label="", seqs=None, window=0, softcap=1.5, scale=None):
    dev = torch.device("cuda")
    q = inp["q"]
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    mask = "sliding" if window else "none"
    announce(f"paged decode {label} {score} window={window}")
    out, lse = af.attn_paged_decode(q.to(dev), inp["k_cache"].to(dev), inp["v_cache"].to(dev),
                                    inp["page_table"].to(dev), inp["seq_lens"].to(dev),
                                    scale=scale, mask=mask, window=window, score=score,
                                    rel_scale=-0.01, softcap=softcap)
    torch.cuda.synchronize()
    ss = oracle.ScoreSpec(workloads.SCORE_NAMES[score], rel_scale=-0.01, softcap=softcap)
    ms = oracle.MaskSpec(workloads.MASK_NAMES[mask], window=window)
    o_ref, l_ref = oracle.paged_decode_ref(f64(q), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                           inp["page_table"].numpy(), inp["seq_lens"].numpy(),
                                           scale, ss, seqs=seqs, mask=ms)
    o = f64(out)
    l = f64(lse)
    if seqs is not None:
        o, l = o[seqs], l[seqs]
    compare(o, l, o_ref, l_ref, torch.bfloat16, label)
    return out, lse


LENGTHS = [1, 15, 16, 17, 1023, 1024, 1025, 1280]


@pytest.mark.parametrize("score", ["none", "alibi", "rel_pos", "softcap"])
def test_paged_decode_small(score):
    run_decode(small_decode_inputs(LENGTHS, seed=1), score, "small")


@pytest.mark.parametrize("softcap", [0.5, 8.0])
def test_paged_decode_softcap_large_scores(softcap):
    # scale 1 over D = 128: scores of spread ~11, saturated by the small cap
    # and bent by cap 8 (a cap far above them would leave a softmax resting
    # on one or two keys, where the bf16 rounding of P and O alone nears the
    # bound)
    run_decode(small_decode_inputs(LENGTHS, seed=4, poison=True), "softcap", "softcap",
               window=300, softcap=softcap, scale=1.0)


def test_paged_decode_nan_poison_and_gqa_groups():
    inp = small_decode_inputs([3, 16, 33, 700, 1100], hq=12, hkv=2, seed=2, poison=True)
    run_decode(inp, "alibi", "poison G=6")
    inp = small_decode_inputs([5, 64, 300], hq=3, hkv=3, seed=3, poison=True)
    run_decode(inp, "none", "poison G=1")


@pytest.mark.parametrize("window", [1, 15, 16, 17, 100, 700, 5000])
def test_paged_decode_sliding_window(window):
    run_decode(small_decode_inputs(LENGTHS, seed=5), "alibi", "window", window=window)


@pytest.mark.parametrize("n_seq,window,split", [(64, 0, 64), (40, 0, 32), (20, 700, 16)])
def test_paged_decode_split_sizes(n_seq, window, split):
    # The launch takes 64-, 32- or 16-page splits depending on how many work
    # items the sequence count, the kv heads and the longest key range give
    # (2048 wanted); these shapes land on each size in turn (20 sequences x 8
    # kv heads are too few items for the one-item-per-sequence form).
    rng = np.random.default_rng(n_seq + window)
    lengths = rng.integers(1, 300 * 16 + 1, size=n_seq)
    lengths[:3] = [0, 1, 300 * 16]
    inp = small_decode_inputs(list(lengths), hq=8, hkv=8, max_pages=300, seed=7)
    run_decode(inp, "alibi", f"split {split}", window=window)


def test_paged_decode_window_skips_pages_before_it():
    # NaN in every slot before each sequence's window: pages wholly before the
    # window are never read, and the keys of the first page that precede the
    # window get no weight.
    lengths = [40, 300, 1100, 1280]
    window = 37
    inp = small_decode_inputs(lengths, hq=8, hkv=2, seed=6, poison=True)
    table = inp["page_table"].numpy()
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    for s, L in enumerate(lengths):
        for t in range(max(0, L - window)):
            inp["k_cache"][table[s, t // 16], :, t % 16] = nan
            inp["v_cache"][table[s, t // 16], :, t % 16] = nan
    run_decode(inp, "none", "window poison", window=window)


def test_paged_decode_many_sequences_and_empty_ones():
    # More sequences than one 64-wide chunk of the work enumeration and empty
    # sequences (O = 0, LSE = -inf).  150 sequences x 2 kv heads over at most
    # 80 pages run as one item per (sequence, kv head), written straight to
    # the output.
    rng = np.random.default_rng(11)
    lengths = [int(x) for x in rng.integers(0, 200, size=150)]
    lengths[0] = 0
    lengths[70] = 0
    lengths[149] = 0
    lengths[5] = 1100
    lengths[100] = 1024
    inp = small_decode_inputs(lengths, hq=8, hkv=2, seed=4)
    run_decode(inp, "alibi", "many sequences")


# One work item per (sequence, kv head), reduced straight into the output,
# when every key range fits 128 pages and there are at least 256 items: 33
# sequences x 8 kv heads, lengths from 0 to 3000, NaN in every slot no
# sequence owns.  Window 2032 is the largest whose range fits 128 pages;
# 2033 takes the split path with the same inputs.
@pytest.mark.parametrize("window", [1, 16, 100, 1024, 2032, 2033])
def test_paged_decode_direct_items(window):
    lengths = [0, 1, 15, 16, 17, 1023, 1024, 1025, 2040, 3000] + [37 * k + 5 for k in range(23)]
    inp = small_decode_inputs(lengths, hq=32, hkv=8, max_pages=200, seed=window, poison=True)
    run_decode(inp, "alibi", "direct items", window=window)


@pytest.mark.parametrize("score", ["none", "rel_pos", "softcap"])
def test_paged_decode_direct_items_scores(score):
    # the other score forms on the direct items (no window: 33 sequences of at
    # most 120 pages, within one item each)
    lengths = [0, 1, 16, 17, 1900] + [53 * k + 7 for k in range(28)]
    inp = small_decode_inputs(lengths, hq=16, hkv=8, max_pages=120, seed=40 + len(score), poison=True)
    run_decode(inp, score, "direct items, no window")


def test_paged_decode_full_workload_sampled():
    w = workloads.PAGED_DECODE
    dev = torch.device("cuda")
    announce("paged decode full workload: generating")
    inp = workloads.decode_inputs(w, device=dev)
    lengths = inp["lengths"]
    scale = 1.0 / math.sqrt(w.D)
    announce("paged decode full workload: run")
    out, lse = af.attn_paged_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                                    inp["seq_lens"], scale=scale)
    out2, lse2 = af.attn_paged_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                                      inp["seq_lens"], scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    seqs = sorted({int(np.argmin(lengths)), int(np.argmax(lengths)), 0, 31, 63})
    table = inp["page_table"].cpu().numpy()
    q = inp["q"].cpu()
    o_ref = np.zeros((len(seqs), w.Hq, w.D))
    l_ref = np.zeros((len(seqs), w.Hq))
    for i, s in enumerate(seqs):
        L = int(lengths[s])
        pages = table[s, :(L + 15) // 16]
        pid = torch.from_numpy(pages.astype(np.int64)).to(dev)
        kc = inp["k_cache"].index_select(0, pid).cpu()
        vc = inp["v_cache"].index_select(0, pid).cpu()
        local = np.arange(len(pages), dtype=np.int32)[None, :]
        o1, l1 = oracle.paged_decode_ref(f64(q[s:s + 1]), f64(kc), f64(vc), local,
                                         np.array([L], dtype=np.int32), scale)
        o_ref[i], l_ref[i] = o1[0], l1[0]
    compare(f64(out)[seqs], f64(lse)[seqs], o_ref, l_ref, torch.bfloat16, "paged decode full")


def test_paged_decode_full_workload_window_alibi_sampled():
    # The 64-sequence workload with a 1024-token window and ALiBi (the
    # PagedAttention + sliding window combination), sampled sequences.
    w = workloads.PAGED_DECODE
    dev = torch.device("cuda")
    announce("paged decode full workload window+alibi: generating")
    inp = workloads.decode_inputs(w, device=dev)
    lengths = inp["lengths"]
    scale = 1.0 / math.sqrt(w.D)
    announce("paged decode full workload window+alibi: run")
    out, lse = af.attn_paged_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                                    inp["seq_lens"], scale=scale, mask="sliding", window=1024,
                                    score="alibi")
    torch.cuda.synchronize()
    seqs = sorted({int(np.argmin(lengths)), int(np.argmax(lengths)), 0, 17, 63})
    table = inp["page_table"].cpu().numpy()
    q = inp["q"].cpu()
    o_ref = np.zeros((len(seqs), w.Hq, w.D))
    l_ref = np.zeros((len(seqs), w.Hq))
    for i, s in enumerate(seqs):
        L = int(lengths[s])
        pages = table[s, :(L + 15) // 16]
        pid = torch.from_numpy(pages.astype(np.int64)).to(dev)
        kc = inp["k_cache"].index_select(0, pid).cpu()
        vc = inp["v_cache"].index_select(0, pid).cpu()
        local = np.arange(len(pages), dtype=np.int32)[None, :]
        o1, l1 = oracle.paged_decode_ref(f64(q[s:s + 1]), f64(kc), f64(vc), local,
                                         np.array([L], dtype=np.int32), scale,
                                         oracle.ScoreSpec(oracle.SCORE_ALIBI),
                                         mask=oracle.MaskSpec(oracle.MASK_SLIDING, window=1024))
        o_ref[i], l_ref[i] = o1[0], l1[0]
    compare(f64(out)[seqs], f64(lse)[seqs], o_ref, l_ref, torch.bfloat16, "paged decode full window")


def test_block_mask_build_into_given_buffers():
    """Building into an existing BlockMask's buffers overwrites every entry:
    a document build over a causal one equals the oracle's document mask."""
    dev = torch.device("cuda")
    B, S = 2, 1000
    doc = torch.from_numpy(_ids([100, 700, 37, 163], B))
    announce("block mask build into given buffers")
    bm = af.attn_build_block_mask("causal", B, S, S, device=dev)
    out = af.attn_build_block_mask("document", B, S, S, doc_ids=doc.to(dev), device=dev, out=bm)
    torch.cuda.synchronize()
    assert out.kv_indices.data_ptr() == bm.kv_indices.data_ptr()
    num, idx, full = oracle.block_mask_ref(oracle.MaskSpec(oracle.MASK_DOCUMENT, doc_ids=doc.numpy()),
                                           B, S, S, 128, 128)
    assert np.array_equal(out.kv_num_blocks.cpu().numpy(), num)
    assert np.array_equal(out.kv_indices.cpu().numpy(), idx)
    assert np.array_equal(out.kv_full.cpu().numpy(), full)
    with pytest.raises(ValueError):
        af.attn_build_block_mask("causal", B, S + 200, S + 200, device=dev, out=bm)
