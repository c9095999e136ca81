"""Top-k softmax router.

Test infrastructure (see the package docstring).

Source: the "FusedMoE Class" section of the overview page gives the layer a
top-K router that feeds the expert kernels; the layer definition fixes it as
a softmax over the E router logits, the k highest-scoring experts per token,
and an optional renormalisation of the k selected weights to sum to one.

Readings where the pages are silent:
  * selection is on the float32 logits (softmax is monotone, so the chosen set
    is the same, and no exp rounding can create or break ties);
  * equal logits go to the lower expert index;
  * slots are ordered by descending score;
  * probabilities are exp(l_e - max l) / sum_i exp(l_i - max l) in float64,
    then (if renormalising) divided by their sum over the k slots, and finally
    rounded to float32.

Pinned by tests/test_oracle_router.py (full-sort brute force, scipy's
softmax, k = E and E = 1 special cases, weight-sum and ordering invariants).
"""

import numpy as np


def topk_softmax(logits, top_k: int, renormalize: bool):
    """logits: float32 [T, E].  Returns (ids int32 [T, k], w float32 [T, k])."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("need 1 <= top_k <= E")
    # stable sort of the negated logits: descending value, ascending index on ties
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :top_k].astype(np.int32)

    l64 = logits.astype(np.float64)
    z = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)
