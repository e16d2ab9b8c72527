"""Gradients of the attention forward: the backward pass from the stored LSE.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[FlexAttention page], introduction: the backward pass is produced by
PyTorch's automatic differentiation of the forward; §性能: the backward is
deterministic and recomputes more intermediates than FlashAttention-2.  The
result is therefore the exact gradient of the forward definition in
attention.py, taken here step by step with the chain rule (reading R22):

    forward:  x = s * Q K^T          (s = fp32 scale)
              S = score_mod(x)       (bias added, or cap * tanh(x / cap))
              S = -inf where hidden
              P = softmax(S)         (rows with no visible key: P = 0)
              O = P V
    given dO (the gradient of a scalar loss with respect to O):
              dV   = P^T dO
              dP   = dO V^T
              D_i  = sum_j P_ij dP_ij = sum_d dO_id O_id
              dS   = P * (dP - D)              (softmax Jacobian, row-wise)
              dX   = dS * score_mod'(x)        (1 for a bias;
                                               1 - tanh^2(x / cap) for the cap)
              dQ   = s * dX K,   dK = s * dX^T Q

With GQA the kv head's dK and dV sum the contributions of every query head
that reads it.  Everything is float64 NumPy with whole score rows
materialised.
"""

from __future__ import annotations

import numpy as np

from . import attention as _att
from .attention import MaskSpec, ScoreSpec, SCORE_SOFTCAP


def _score_mod_grad(score: ScoreSpec, x: np.ndarray) -> np.ndarray:
    """d score_mod(x) / dx elementwise: 1 for the additive kinds, and
    1 - tanh^2(x / cap) for soft-capping."""
    if score.kind == SCORE_SOFTCAP:
        t = np.tanh(x / float(score.softcap))
        return 1.0 - t * t
    return np.ones_like(x)


def attention_backward_rows(q_rows, k, v, do_rows, row_idx, b: int, hq: int, hq_count: int, scale,
                            mask: MaskSpec = MaskSpec(), score: ScoreSpec = ScoreSpec()):
    """(dQ rows, dK contribution, dV contribution) of some query rows of one
    (b, hq) against all keys k, v [m, D].  Float64."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do_rows = np.asarray(do_rows, dtype=np.float64)
    s_fp = _att._fp32_scale(scale)
    x = s_fp * (q_rows @ k.T)
    s = _att.scores_block(q_rows, k, scale, mask, score, b, hq, hq_count, row_idx)
    p, _, _ = _att.softmax_safe3(s)
    o = p @ v
    dv = p.T @ do_rows
    dp = do_rows @ v.T
    d_row = np.sum(do_rows * o, axis=1)
    ds = p * (dp - d_row[:, None])
    dx = ds * _score_mod_grad(score, x)
    dq = s_fp * (dx @ k)
    dk = s_fp * (dx.T @ q_rows)
    return dq, dk, dv


def attention_backward_ref(q, k, v, dout, scale, mask: MaskSpec = MaskSpec(),
                           score: ScoreSpec = ScoreSpec(), row_block: int = 1024):
    """dQ [B,Hq,Sq,D], dK [B,Hkv,Skv,D], dV [B,Hkv,Skv,Dv] (float64) of the
    loss whose gradient with respect to O is dout [B,Hq,Sq,Dv]."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    bsz, hq_count, sq, _ = q.shape
    hkv_count = k.shape[1]
    if hq_count % hkv_count != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    rows = np.arange(sq)
    for b in range(bsz):
        for hq in range(hq_count):
            hkv = _att.kv_head(hq, hq_count, hkv_count)
            for r0 in range(0, sq, row_block):
                ridx = rows[r0:r0 + row_block]
                dq_r, dk_c, dv_c = attention_backward_rows(q[b, hq][ridx], k[b, hkv], v[b, hkv],
                                                           dout[b, hq][ridx], ridx, b, hq, hq_count,
                                                           scale, mask, score)
                dq[b, hq, ridx] = dq_r
                dk[b, hkv] += dk_c
                dv[b, hkv] += dv_c
    return dq, dk, dv


def softmax_row_dot_ref(out, dout):
    """D = rowsum(dO * O) [B, Hq, Sq], the per-row term of the softmax
    Jacobian, in float64."""
    return np.sum(np.asarray(out, dtype=np.float64) * np.asarray(dout, dtype=np.float64), axis=-1)
