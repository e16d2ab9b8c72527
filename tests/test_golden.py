"""Closed-form values of the workloads (tests/golden/workload_closed_forms.json).

The pages print no worked numeric example, so the stored values are
derivations from the mask definitions (FlexAttention page: intro variant list,
§Causal Mask, §Sliding Window + Causal) and the seeded input recipe.  Each
value is re-derived here by its own formula, then the oracle's BlockMask, the
seeded generators and the bench's FLOP basis are checked against it.
"""

import json
import os

import numpy as np

import oracle
import workloads
from oracle import MaskSpec, MASK_CAUSAL, MASK_SLIDING, MASK_DOCUMENT, MASK_AND

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "workload_closed_forms.json")))


def test_visible_pairs_closed_forms():
    g = GOLDEN["visible_pairs_per_head"]
    assert g["dense_s2048"]["value"] == 2048 ** 2
    assert g["causal_s2048"]["value"] == 2048 * 2049 // 2
    s, w = 8192, 1024
    assert g["sliding_s8192_w1024"]["value"] == w * (w + 1) // 2 + (s - w) * w
    lengths = GOLDEN["seeded_structure"]["doc_lengths_seed0"]
    assert sum(lengths) == 16384
    assert g["document_s16384_seed0"]["value"] == sum(n * (n + 1) // 2 for n in lengths)


def test_bench_flop_basis_matches():
    import bench
    g = GOLDEN["visible_pairs_per_head"]
    assert bench.visible_pairs("none", 2048) == g["dense_s2048"]["value"]
    assert bench.visible_pairs("causal", 2048) == g["causal_s2048"]["value"]
    assert bench.visible_pairs("sliding", 8192, 1024) == g["sliding_s8192_w1024"]["value"]
    lengths = GOLDEN["seeded_structure"]["doc_lengths_seed0"]
    assert bench.visible_pairs("document", 16384, doc_lengths=lengths) == g["document_s16384_seed0"]["value"]


def test_oracle_visible_count_matches_on_small_rows():
    # The oracle's predicate summed over a few whole rows equals the closed
    # form restricted to those rows.
    s, w = 8192, 1024
    rows = np.array([0, 1, 1023, 1024, 5000, s - 1])
    j = np.arange(s)
    got = sum(int(oracle.visible(MaskSpec(MASK_SLIDING, window=w), 0, np.array([i]), j).sum()) for i in rows)
    assert got == sum(min(i + 1, w) for i in rows)


def test_block_mask_counts():
    g = GOLDEN["block_mask_128"]
    num, _, full = oracle.block_mask_ref(MaskSpec(MASK_CAUSAL), 1, 2048, 2048, 128, 128)
    n = 16
    assert (g["causal_s2048"]["listed"], g["causal_s2048"]["full"]) == (n * (n + 1) // 2, n * (n - 1) // 2)
    assert (int(num.sum()), int(full.sum())) == (g["causal_s2048"]["listed"], g["causal_s2048"]["full"])
    num, _, full = oracle.block_mask_ref(MaskSpec(MASK_SLIDING, window=1024), 1, 8192, 8192, 128, 128)
    n = 64
    assert g["sliding_s8192_w1024"]["listed"] == sum(min(qb + 1, 9) for qb in range(n))
    assert g["sliding_s8192_w1024"]["full"] == sum(min(qb, 7) for qb in range(n))
    assert (int(num.sum()), int(full.sum())) == (g["sliding_s8192_w1024"]["listed"],
                                                 g["sliding_s8192_w1024"]["full"])
    lengths = GOLDEN["seeded_structure"]["doc_lengths_seed0"]
    ids = np.repeat(np.arange(len(lengths)), lengths)[None, :]
    num, _, full = oracle.block_mask_ref(MaskSpec(MASK_DOCUMENT, doc_ids=ids), 1, 16384, 16384, 128, 128)
    assert (int(num.sum()), int(full.sum())) == (g["document_s16384_seed0"]["listed"],
                                                 g["document_s16384_seed0"]["full"])


def test_seeded_generators():
    s = GOLDEN["seeded_structure"]
    assert workloads.doc_lengths(16384, 256, 4096, seed=0) == s["doc_lengths_seed0"]
    lengths, _ = workloads.decode_lengths(64, 1024, 32768, seed=0)
    d = s["decode_lengths_seed0"]
    assert (int(np.sum(lengths)), int(np.min(lengths)), int(np.max(lengths))) == (d["sum"], d["min"], d["max"])
    assert int(sum(-(-int(L) // 16) for L in lengths)) == d["pool_pages"]
    kv = int(np.sum(lengths)) * 2 * 8 * 128 * 2
    total = kv + 2 * 64 * 32 * 128 * 2 + 64 * 32 * 4 + d["pool_pages"] * 4 + 64 * 4
    assert total == s["decode_algorithmic_bytes"]["value"]


def _doc_window_pairs(lengths, w):
    return sum(n * (n + 1) // 2 if n <= w else w * (w + 1) // 2 + (n - w) * w for n in lengths)


def test_document_window_closed_forms():
    # sliding window 1024 + document + causal over the seed-0 documents
    lengths = GOLDEN["seeded_structure"]["doc_lengths_seed0"]
    g = GOLDEN["visible_pairs_per_head"]["document_window1024_s16384_seed0"]
    assert g["value"] == _doc_window_pairs(lengths, 1024)
    import bench
    assert bench.visible_pairs("sliding&document&causal", 16384, 1024, doc_lengths=lengths) == g["value"]
    # the oracle's predicate on whole rows: each row sees min(i - start + 1, W) keys
    ids = workloads.doc_ids_from_lengths(lengths, 1)
    m = MaskSpec(MASK_AND, window=1024, doc_ids=ids, and_kinds=(MASK_SLIDING, MASK_DOCUMENT, MASK_CAUSAL))
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    rows = [0, 1, 1100, 3522, 3523, 3524, 3523 + 1500, 16383]
    j = np.arange(16384)
    for i in rows:
        st = starts[np.searchsorted(starts, i, side="right") - 1]
        assert int(oracle.visible(m, 0, np.array([i]), j).sum()) == min(i - st + 1, 1024)
    # block counts: interval test per document (the derivation stored with them)
    bm = GOLDEN["block_mask_128"]["document_window1024_s16384_seed0"]
    ends = starts + np.array(lengths)
    listed = full = 0
    for qb in range(128):
        q0, q1 = 128 * qb, 128 * qb + 127
        for kb in range(128):
            k0, k1 = 128 * kb, 128 * kb + 127
            li = fu = False
            for s0, e0 in zip(starts, ends):
                a, b = max(q0, s0), min(q1, e0 - 1)
                c, d = max(k0, s0), min(k1, e0 - 1)
                if a > b or c > d:
                    continue
                li |= (b - c >= 0) and (a - d < 1024)
                fu |= s0 <= min(q0, k0) and e0 - 1 >= max(q1, k1) and q0 - k1 >= 0 and q1 - k0 < 1024
            listed += li
            full += fu
    assert (listed, full) == (bm["listed"], bm["full"])
    num, _, fl = oracle.block_mask_ref(m, 1, 16384, 16384, 128, 128)
    assert (int(num.sum()), int(fl.sum())) == (bm["listed"], bm["full"])
