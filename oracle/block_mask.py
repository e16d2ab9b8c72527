"""Block-sparse mask (BlockMask) reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[FlexAttention page], introduction: the system exploits the sparsity of the
attention mask to beat standard attention.  The page gives no layout; the one
taken here:

* the Sq x Skv visibility grid is cut into q_block x kv_block blocks, the
  last row / column of blocks clipped at Sq / Skv;
* for every (b, query block qb) the key blocks kb that hold at least one
  visible (i, j) are listed in ascending order in kv_indices[b, 0, qb, :],
  their number in kv_num_blocks[b, 0, qb];
* kv_full[b, 0, qb, n] = 1 when every (i, j) of the listed block is visible
  (the kernel may then skip the per-element predicate);
* unused tail entries are kv_indices = -1 and kv_full = 0;
* the head axis has size 1: no mask kind here depends on the head;
* the backward also needs the lists the other way round, per key block the
  ascending query blocks (block_mask_cols_ref): the same (block, block)
  incidence, transposed.

Only the mask decides sparsity (no score modifier produces -inf).
"""

from __future__ import annotations

import numpy as np

from .attention import MaskSpec, visible, MASK_NONE, MASK_CAUSAL, MASK_SLIDING, \
    MASK_PREFIX_LM, MASK_DOCUMENT, MASK_AND


def block_mask_ref(mask: MaskSpec, batch: int, sq: int, skv: int,
                   q_block: int = 128, kv_block: int = 128):
    """Returns (kv_num_blocks int32 [B,1,nQB], kv_indices int32 [B,1,nQB,nKVB],
    kv_full uint8 [B,1,nQB,nKVB]) from the element-wise visibility grid."""
    nqb = -(-sq // q_block)
    nkb = -(-skv // kv_block)
    num = np.zeros((batch, 1, nqb), dtype=np.int32)
    idx = np.full((batch, 1, nqb, nkb), -1, dtype=np.int32)
    full = np.zeros((batch, 1, nqb, nkb), dtype=np.uint8)
    cols = np.arange(skv)
    for b in range(batch):
        for qb in range(nqb):
            rows = np.arange(qb * q_block, min(sq, (qb + 1) * q_block))
            vis = visible(mask, b, rows, cols)
            n = 0
            for kb in range(nkb):
                blk = vis[:, kb * kv_block:min(skv, (kb + 1) * kv_block)]
                if blk.any():
                    idx[b, 0, qb, n] = kb
                    full[b, 0, qb, n] = 1 if blk.all() else 0
                    n += 1
            num[b, 0, qb] = n
    return num, idx, full


def block_mask_cols_ref(mask: MaskSpec, batch: int, sq: int, skv: int,
                        q_block: int = 128, kv_block: int = 128):
    """The same blocks listed by key block, for the backward's key-stationary
    pass: (q_num_blocks int32 [B,1,nKVB], q_indices int32 [B,1,nKVB,nQB]
    ascending with -1 tails, q_full uint8 [B,1,nKVB,nQB] with 0 tails), from
    the element-wise visibility grid."""
    nqb = -(-sq // q_block)
    nkb = -(-skv // kv_block)
    num = np.zeros((batch, 1, nkb), dtype=np.int32)
    idx = np.full((batch, 1, nkb, nqb), -1, dtype=np.int32)
    full = np.zeros((batch, 1, nkb, nqb), dtype=np.uint8)
    rows = np.arange(sq)
    for b in range(batch):
        for kb in range(nkb):
            cols = np.arange(kb * kv_block, min(skv, (kb + 1) * kv_block))
            vis = visible(mask, b, rows, cols)
            n = 0
            for qb in range(nqb):
                blk = vis[qb * q_block:min(sq, (qb + 1) * q_block), :]
                if blk.any():
                    idx[b, 0, kb, n] = qb
                    full[b, 0, kb, n] = 1 if blk.all() else 0
                    n += 1
            num[b, 0, kb] = n
    return num, idx, full


def block_mask_bruteforce(kind: int, batch: int, sq: int, skv: int, q_block: int,
                          kv_block: int, window: int = 0, prefix_len: int = 0, doc_ids=None,
                          and_kinds=()):
    """Element-by-element scalar form for tiny shapes (pure Python)."""
    doc = None if doc_ids is None else np.asarray(doc_ids).tolist()

    def vis(b, i, j, kind=kind):
        if kind == MASK_NONE:
            return True
        if kind == MASK_CAUSAL:
            return j <= i
        if kind == MASK_SLIDING:
            return 0 <= i - j < window
        if kind == MASK_PREFIX_LM:
            return j <= i or j < prefix_len
        if kind == MASK_DOCUMENT:
            return doc[b][i] == doc[b][j] and j <= i
        if kind == MASK_AND:
            return all(vis(b, i, j, part) for part in and_kinds)
        raise ValueError(kind)

    nqb = -(-sq // q_block)
    nkb = -(-skv // kv_block)
    num = [[[0] * nqb] for _ in range(batch)]
    idx = [[[[-1] * nkb for _ in range(nqb)]] for _ in range(batch)]
    full = [[[[0] * nkb for _ in range(nqb)]] for _ in range(batch)]
    for b in range(batch):
        for qb in range(nqb):
            n = 0
            for kb in range(nkb):
                seen = 0
                total = 0
                for i in range(qb * q_block, min(sq, (qb + 1) * q_block)):
                    for j in range(kb * kv_block, min(skv, (kb + 1) * kv_block)):
                        total += 1
                        seen += 1 if vis(b, i, j) else 0
                if seen:
                    idx[b][0][qb][n] = kb
                    full[b][0][qb][n] = 1 if seen == total else 0
                    n += 1
            num[b][0][qb] = n
    return (np.array(num, dtype=np.int32), np.array(idx, dtype=np.int32),
            np.array(full, dtype=np.uint8))
