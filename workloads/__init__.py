"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and integer structure; it holds none of
the attention arithmetic, so the oracle and the HIP path can both be fed from
it without sharing any computation.

Recipe (the pages measure no public benchmark for this path; every input is
synthetic):
* float tensors: ``torch.Generator(device).manual_seed(seed)``, then q, k, v
  drawn in that order with ``torch.randn(..., dtype=float32)`` (i.i.d.
  N(0, 1)), cast to bf16 (round to nearest even) for bf16 workloads;
* document lengths: ``numpy.random.default_rng(seed).integers(lo, hi,
  endpoint=True)`` drawn until the running total reaches the packed length,
  the last document truncated to fit;
* decode KV lengths: ``default_rng(seed).integers(lo, hi, size=N,
  endpoint=True)``; the page pool holds exactly sum ceil(L/16) pages and the
  page table hands each sequence, in order, the next entries of
  ``rng.permutation(pool)`` (same rng, next draw); unused entries are -1;
* the decode K/V pool is drawn on the device it will live on (2 x 2.26 GB in
  bf16 at the full shape), chunk by chunk from one seeded generator.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

MASK_NAMES = {"none": 0, "causal": 1, "sliding": 2, "prefix_lm": 3, "document": 4}
SCORE_NAMES = {"none": 0, "alibi": 1, "rel_pos": 2, "softcap": 3}


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    dtype: str              # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    mask: str = "none"
    score: str = "none"
    window: int = 0
    prefix_len: int = 0
    softcap: float = 0.0    # score "softcap": the cap
    docs: bool = False      # document ids drawn with doc_lengths()
    block_mask: bool = False
    seed: int = 0


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    Hq: int
    Hkv: int
    D: int
    page_size: int = 16
    len_lo: int = 1024
    len_hi: int = 32768
    max_pages: int = 2048
    seed: int = 0


# The five workloads the measurements and parity cases are defined on.
TINY_CAUSAL_F32 = PrefillWorkload("tiny_causal_f32_b1h2s128d64", "f32", 1, 2, 2, 128, 128, 64,
                                  mask="causal")
DENSE_BF16 = PrefillWorkload("dense_bf16_b4h16s2048d64", "bf16", 4, 16, 16, 2048, 2048, 64)
CAUSAL_BF16 = PrefillWorkload("causal_bf16_b4h16s2048d64", "bf16", 4, 16, 16, 2048, 2048, 64,
                              mask="causal")
GQA_WINDOW_ALIBI = PrefillWorkload("gqa_window1024_alibi_bf16_b2hq32hkv8s8192d128", "bf16",
                                   2, 32, 8, 8192, 8192, 128, mask="sliding", score="alibi",
                                   window=1024)
DOCUMENT_BLOCKMASK = PrefillWorkload("document_blockmask_bf16_b1h16s16384d128", "bf16",
                                     1, 16, 16, 16384, 16384, 128, mask="document", docs=True,
                                     block_mask=True)
# The pages' combination sliding window + document + causal, intersected,
# on the document workload's shape and documents.
DOC_WINDOW_BLOCKMASK = PrefillWorkload("document_window1024_blockmask_bf16_b1h16s16384d128", "bf16",
                                       1, 16, 16, 16384, 16384, 128, mask="sliding&document&causal",
                                       window=1024, docs=True, block_mask=True)
# The causal shape again with soft-capping; N(0, 1) inputs give scaled scores
# of unit spread, so a cap of 5 bends their tails as larger caps do on
# trained logits.
CAUSAL_SOFTCAP = PrefillWorkload("causal_softcap5_bf16_b4h16s2048d64", "bf16", 4, 16, 16, 2048, 2048,
                                 64, mask="causal", score="softcap", softcap=5.0)
PAGED_DECODE = DecodeWorkload("paged_decode_bf16_n64hq32hkv8d128p16", 64, 32, 8, 128)
# Longer launches of the same kernel, for scale only (timed, not parity
# workloads): the GQA shape without window or bias, dense and causal, and the
# dense D=64 shape at S=8192.
LONG_DENSE_D128 = PrefillWorkload("long_dense_bf16_b2hq32hkv8s8192d128", "bf16", 2, 32, 8, 8192, 8192, 128)
LONG_CAUSAL_D128 = PrefillWorkload("long_causal_bf16_b2hq32hkv8s8192d128", "bf16", 2, 32, 8, 8192, 8192,
                                   128, mask="causal")
LONG_DENSE_D64 = PrefillWorkload("long_dense_bf16_b2h32s8192d64", "bf16", 2, 32, 32, 8192, 8192, 64)

PREFILL_WORKLOADS = [TINY_CAUSAL_F32, DENSE_BF16, CAUSAL_BF16, GQA_WINDOW_ALIBI, DOCUMENT_BLOCKMASK,
                     CAUSAL_SOFTCAP, DOC_WINDOW_BLOCKMASK]


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def randn_qkv(B, Hq, Hkv, Sq, Skv, D, dtype: str = "bf16", seed: int = 0, device="cpu"):
    """q [B,Hq,Sq,D], k and v [B,Hkv,Skv,D], drawn q, k, v in that order."""
    g = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn((B, Hq, Sq, D), dtype=torch.float32, generator=g, device=device)
    k = torch.randn((B, Hkv, Skv, D), dtype=torch.float32, generator=g, device=device)
    v = torch.randn((B, Hkv, Skv, D), dtype=torch.float32, generator=g, device=device)
    dt = torch_dtype(dtype)
    return q.to(dt), k.to(dt), v.to(dt)


def doc_lengths(total: int = 16384, lo: int = 256, hi: int = 4096, seed: int = 0):
    """Document lengths uniform in [lo, hi] until the total is reached; the
    last one truncated so the lengths sum to exactly `total`."""
    rng = np.random.default_rng(seed)
    lengths = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, total - acc)
        lengths.append(n)
        acc += n
    return lengths


def doc_ids_from_lengths(lengths, batch: int = 1):
    """int32 [batch, sum(lengths)]: token t of document d gets id d."""
    ids = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)
    return np.tile(ids[None, :], (batch, 1)).astype(np.int32)


def prefill_inputs(w: PrefillWorkload, device="cpu"):
    """Everything a prefill workload needs, on `device` (doc ids as int32)."""
    q, k, v = randn_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, w.dtype, w.seed, device)
    out = {"q": q, "k": k, "v": v, "doc_ids": None, "doc_lengths": None}
    if w.docs:
        lengths = doc_lengths(w.Sq, seed=w.seed)
        out["doc_lengths"] = lengths
        out["doc_ids"] = torch.from_numpy(doc_ids_from_lengths(lengths, w.B)).to(device)
    return out


def decode_lengths(n: int = 64, lo: int = 1024, hi: int = 32768, seed: int = 0):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi, size=n, endpoint=True).astype(np.int64)
    return lengths, rng


def decode_page_table(lengths, rng, page_size: int = 16, max_pages: int = 2048):
    """(page_table int32 [N, max_pages] with -1 tails, pool size in pages)."""
    pages_per = [-(-int(L) // page_size) for L in lengths]
    pool = int(sum(pages_per))
    if max(pages_per) > max_pages:
        raise ValueError("max_pages too small for the drawn lengths")
    perm = rng.permutation(pool).astype(np.int32)
    table = np.full((len(lengths), max_pages), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(pages_per):
        table[s, :n] = perm[pos:pos + n]
        pos += n
    return table, pool


def decode_inputs(w: DecodeWorkload, device="cpu", chunk_pages: int = 4096,
                  lengths: Optional[np.ndarray] = None):
    """q [N,Hq,D] bf16, k_cache / v_cache [pool,Hkv,page,D] bf16, page_table
    int32 [N,max_pages], seq_lens int32 [N]; all on `device`."""
    if lengths is None:
        lengths, rng = decode_lengths(w.N, w.len_lo, w.len_hi, w.seed)
    else:
        rng = np.random.default_rng(w.seed)
        lengths = np.asarray(lengths, dtype=np.int64)
    table, pool = decode_page_table(lengths, rng, w.page_size, w.max_pages)
    g = torch.Generator(device=device).manual_seed(w.seed)
    q = torch.randn((w.N, w.Hq, w.D), dtype=torch.float32, generator=g, device=device)
    q = q.to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = torch.empty((pool, w.Hkv, w.page_size, w.D), dtype=torch.bfloat16, device=device)
        for p0 in range(0, pool, chunk_pages):
            p1 = min(pool, p0 + chunk_pages)
            c[p0:p1] = torch.randn((p1 - p0, w.Hkv, w.page_size, w.D), dtype=torch.float32,
                                   generator=g, device=device).to(torch.bfloat16)
        caches.append(c)
    return {
        "q": q, "k_cache": caches[0], "v_cache": caches[1],
        "page_table": torch.from_numpy(table).to(device),
        "seq_lens": torch.from_numpy(lengths.astype(np.int32)).to(device),
        "lengths": lengths, "pool": pool,
    }
