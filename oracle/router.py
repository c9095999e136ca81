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

Grouped top-k (grouped_topk_softmax).  The overview page's environment table
names a fused grouped top-K routing switch and gives no definition; the
plainest reading, in the router's own terms: the E experts form
num_expert_group equal groups of consecutive ids; a group's score is its best
logit; the topk_group best groups are kept (ties to the lower group index);
the top_k experts are then chosen as above among the kept groups' experts
only.  The weights are the same full softmax over all E logits, renormalised
over the chosen slots if asked: grouping limits which experts may be chosen,
not how they are scored.  Pinned by brute force, by its reduction to the
plain router (one group, or every group kept) and by the group-count
invariant.
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


def grouped_topk_softmax(logits, top_k: int, num_expert_group: int, topk_group: int,
                         renormalize: bool):
    """logits float32 [T, E], E divisible by num_expert_group, 1 <= topk_group
    <= num_expert_group, top_k <= topk_group * (E / num_expert_group).
    Returns (ids int32 [T, k], w float32 [T, k])."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    G = num_expert_group
    if G < 1 or E % G or not 1 <= topk_group <= G or not 1 <= top_k <= topk_group * (E // G):
        raise ValueError("invalid grouping")
    gs = E // G
    gscore = logits.reshape(T, G, gs).max(axis=2)
    gorder = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]
    keep = np.zeros((T, G), dtype=bool)
    np.put_along_axis(keep, gorder, True, axis=1)
    allowed = np.repeat(keep, gs, axis=1)
    masked = np.where(allowed, logits, -np.inf)
    order = np.argsort(-masked, axis=1, kind="stable")
    ids = order[:, :top_k].astype(np.int32)

    l64 = logits.astype(np.float64)
    z = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)
