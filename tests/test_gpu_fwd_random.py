"""Seeded random forward and backward cases against the CPU float64 oracle,
through the C ABI.

Each case draws its own shape and options: batch, head grouping (groups of 1
to 8, including the four-head workgroups and a head count that does not fill
the 8 XCDs evenly), head dim, mask kind or AND of kinds, score modifier,
ragged and rectangular lengths, window, prefix length, document lengths, and
the BlockMask or the analytic key range.  The draws are fixed by the case
number, so a failure names a reproducible case.
"""

import numpy as np
import pytest

from gpu_util import has_document, requires_gpu
from test_gpu_fwd import run_case

pytestmark = [pytest.mark.gpu, requires_gpu]

HEADS = [(1, 1), (2, 1), (4, 1), (4, 2), (8, 2), (8, 1), (12, 3), (16, 4)]
MASKS = ["none", "causal", "sliding", "prefix_lm", "document", "sliding&document&causal", "causal&sliding"]
SCORES = ["none", "alibi", "rel_pos", "softcap"]


def draw(case: int):
    rng = np.random.default_rng(1000 + case)
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    mask = MASKS[rng.integers(len(MASKS))]
    score = SCORES[rng.integers(len(SCORES))]
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    Sq = int(rng.integers(1, 520))
    Skv = Sq if (has_document(mask) or rng.random() < 0.5) else int(rng.integers(1, 520))
    window = int(rng.integers(1, 600))
    prefix_len = int(rng.integers(0, 400))
    n_docs = int(rng.integers(1, 6))
    cuts = np.sort(rng.choice(np.arange(1, max(Sq, 2)), size=min(n_docs - 1, max(Sq - 1, 0)), replace=False))
    lens = tuple(int(x) for x in np.diff(np.concatenate([[0], cuts, [Sq]])) if x > 0) or (Sq,)
    block_mask = bool(rng.random() < 0.4)
    return dict(B=B, Hq=hq, Hkv=hkv, Sq=Sq, Skv=Skv, D=D, mask=mask, score=score, window=window,
                prefix_len=prefix_len, doc_lengths=lens, block_mask=block_mask, seed=case)


@pytest.mark.parametrize("case", range(64))
def test_bf16_random_case(case):
    c = draw(case)
    run_case(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Skv"], c["D"], "bf16", c["mask"], c["score"],
             seed=c["seed"], window=c["window"], prefix_len=c["prefix_len"], doc_lengths=c["doc_lengths"],
             block_mask=c["block_mask"], mha_equal=(c["Hq"] // c["Hkv"]) % 4 == 0 and not c["block_mask"])


@pytest.mark.parametrize("case", range(16))
def test_bwd_random_case(case):
    from test_gpu_bwd import run_bwd
    c = draw(500 + case)
    Sq = min(c["Sq"], 300)
    Skv = Sq if c["Skv"] == c["Sq"] else min(c["Skv"], 300)
    lens = list(c["doc_lengths"])
    # document lengths re-cut to the shortened Sq
    if sum(lens) > Sq:
        acc, cut = 0, []
        for x in lens:
            if acc + x >= Sq:
                cut.append(Sq - acc)
                break
            cut.append(x)
            acc += x
        lens = [x for x in cut if x > 0]
    run_bwd(c["B"], c["Hq"], c["Hkv"], Sq, Skv, c["D"], c["mask"], c["score"], seed=c["seed"],
            window=c["window"], prefix_len=c["prefix_len"], doc_lengths=tuple(lens),
            block_mask=c["block_mask"])
