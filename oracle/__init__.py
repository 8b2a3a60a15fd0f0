"""CPU fp64 oracle for the fused exact attention forward.

TEST INFRASTRUCTURE. Only the test-suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package. The GPU library never calls it, shares no code with it and has
no CPU fallback through it.

What it computes is the plain definition of scaled dot-product attention with
an additive bias, written out in float64 with the score matrix S and the
probability matrix P materialised (the "standard attention" that the pages set
against the fused kernel):

    S = scale * Q K^T + B,   P = softmax_row(S),   O = P V,
    LSE_i = log sum_j exp(S_ij)

[Understanding FlashAttention Pt 1: Personal Notes, §0.2 "Notation" and §1.1;
 flash-attention (stanleyjacob.dev), Part VI, for the log-sum-exp output.]

Besides the definition it holds the two streaming forms the pages derive
(one key at a time, and blockwise), and the merge of partial (O, LSE) pairs;
the tests pin the definition against those and against worked numbers printed
on the pages.

Every function here is pinned by a test under ``tests/`` (see
``tests/test_oracle_pins.py``); none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    attention_rows,
    attention_varlen,
    score_matrix,
    masked_softmax,
    online_softmax_scalar,
    online_softmax_blocked,
    merge_partials,
)
