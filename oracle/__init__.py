"""CPU float64 oracle for fused attention forward, BlockMask construction and
paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers,
tables or helpers with the HIP library; the two meet only at the seeded input
generators in ``workloads/``, which hold none of the method's arithmetic.

Every function here is the plain definition written out in float64 with
NumPy: the full score matrix (per block of whole rows) is materialised, the
bias and the mask are applied explicitly, and softmax is taken in three passes
(max, sum, normalise).  Library primitives used as single steps: NumPy's
matrix product (BLAS dgemm), ``np.exp``, ``np.log``.

Sources (cited by page title and section; the pages' formulas were images and
are lost, so each reading taken is stated where it is used):

* [FlexAttention page] "新PyTorch API：几行代码实现不同注意力变体，兼具
  FlashAttention性能和PyTorch灵活性" (17aitech.com): the variant list in the
  introduction; §FlexAttention (softmax attention, the per-score
  ``score_mod(score, b, h, q_idx, kv_idx)`` applied before softmax, and the
  five-deep loop that defines it); §全注意力 (identity score_mod);
  §相对位置编码 (bias from the query-key distance, computed in-kernel);
  §Soft-capping (named, formula lost); §Causal Mask; the combination
  sliding window + document + causal in the variant list (AND of masks);
  the backward by automatic differentiation (intro) and its deterministic,
  recomputing algorithm (§性能); §Sliding Window + Causal (the most recent 1024 tokens).
* [Online-Softmax page] "Attention优化｜2w字原理&图解: 从Online-Softmax到
  FlashAttention V1/V2/V3", abstract: 3-pass safe softmax, 2-pass online
  softmax and 1-pass FlashAttention are forms of one result.
* [Pallas page] "高级特性：探索PyTorch/XLA的Pallas内核和Flash Attention实现":
  a multi-query paged-attention kernel (the paged-decode workload).
* [PyTorch 2.0 page] PyTorch 2.0 release news, §概括: the
  ``scaled_dot_product_attention`` operator (used only as an independent
  library cross-check in the tests).

Parity status of each function is recorded in its docstring: every public
function is pinned by the ``-m "not gpu"`` tests (closed forms, brute force,
invariants, library cross-checks); none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    MASK_NONE, MASK_CAUSAL, MASK_SLIDING, MASK_PREFIX_LM, MASK_DOCUMENT, MASK_AND,
    SCORE_NONE, SCORE_ALIBI, SCORE_REL_POS, SCORE_SOFTCAP,
    MaskSpec, ScoreSpec,
    alibi_slopes, visible, bias, score_mod, scores_block, kv_head,
    softmax_naive, softmax_safe3, softmax_online2,
    attention_rows, attention_ref, attention_bruteforce, attention_one_pass,
)
from .block_mask import block_mask_ref, block_mask_cols_ref, block_mask_bruteforce  # noqa: F401
from .backward import attention_backward_ref, attention_backward_rows, softmax_row_dot_ref  # noqa: F401
from .paged_decode import (  # noqa: F401
    gather_paged_kv, paged_decode_ref, split_partials_ref, lse_combine_ref,
)
