"""Pins of oracle/router.py: a full-sort brute force with explicit
tie-breaking, scipy's softmax, and the special cases k = E and E = 1."""

import numpy as np
import pytest
from scipy.special import softmax

from oracle import router


def _brute(logits, k, renorm):
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        ids[t] = order[:k]
        p = softmax(logits[t].astype(np.float64))
        sel = p[order[:k]]
        w[t] = sel / sel.sum() if renorm else sel
    return ids, w


@pytest.mark.parametrize("T,E,k", [(7, 8, 2), (5, 16, 8), (3, 256, 8), (4, 5, 5), (2, 1, 1)])
@pytest.mark.parametrize("renorm", [True, False])
def test_brute_force(T, E, k, renorm):
    rng = np.random.default_rng(T * E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = router.topk_softmax(logits, k, renorm)
    bids, bw = _brute(logits, k, renorm)
    assert np.array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=1e-7, atol=0)
    assert w.dtype == np.float32 and ids.dtype == np.int32


def test_ties_go_to_lower_index():
    logits = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]], dtype=np.float32)
    ids, w = router.topk_softmax(logits, 3, True)
    assert ids.tolist() == [[1, 2, 4]]
    np.testing.assert_allclose(w, [[1 / 3, 1 / 3, 1 / 3]], rtol=1e-7)
    ids, _ = router.topk_softmax(np.zeros((1, 6), np.float32), 2, False)
    assert ids.tolist() == [[0, 1]]


def test_invariants():
    rng = np.random.default_rng(4)
    logits = (rng.standard_normal((200, 128)) * 3).astype(np.float32)
    ids, w = router.topk_softmax(logits, 8, True)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.all(np.diff(w, axis=1) <= 0)                 # descending slots
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    rest = np.sort(logits, axis=1)[:, ::-1][:, 8:]
    assert np.all(sel.min(axis=1) >= rest.max(axis=1))     # top-k by logit


def test_k_equals_e_is_plain_softmax():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((4, 6)).astype(np.float32)
    ids, w = router.topk_softmax(logits, 6, True)
    p = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-7)


def test_single_expert():
    ids, w = router.topk_softmax(np.array([[2.5], [-1.0]], np.float32), 1, False)
    assert ids.tolist() == [[0], [0]] and w.tolist() == [[1.0], [1.0]]


def test_bad_k():
    with pytest.raises(ValueError):
        router.topk_softmax(np.zeros((1, 4), np.float32), 5, True)


# ---- grouped top-k ----

def _brute_grouped(logits, k, G, kg, renorm):
    T, E = logits.shape
    gs = E // G
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    for t in range(T):
        best = []
        for g in range(G):
            m = max(float(logits[t, e]) for e in range(g * gs, (g + 1) * gs))
            best.append((-m, g))
        kept = {g for _, g in sorted(best)[:kg]}
        cand = [e for e in range(E) if e // gs in kept]
        order = sorted(cand, key=lambda e: (-float(logits[t, e]), e))
        ids[t] = order[:k]
        p = softmax(logits[t].astype(np.float64))
        sel = p[order[:k]]
        w[t] = sel / sel.sum() if renorm else sel
    return ids, w


@pytest.mark.parametrize("T,E,k,G,kg", [(6, 16, 4, 4, 2), (5, 256, 8, 8, 4), (4, 64, 6, 8, 3),
                                        (3, 32, 2, 32, 2), (4, 12, 3, 3, 1)])
@pytest.mark.parametrize("renorm", [True, False])
def test_grouped_brute_force(T, E, k, G, kg, renorm):
    rng = np.random.default_rng(T * E + k * G + kg)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :] = np.round(logits[0, :])          # ties inside and across groups
    ids, w = router.grouped_topk_softmax(logits, k, G, kg, renorm)
    bids, bw = _brute_grouped(logits, k, G, kg, renorm)
    assert np.array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=1e-7, atol=0)


def test_grouped_reduces_to_plain_router():
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((20, 64)).astype(np.float32)
    plain = router.topk_softmax(logits, 8, True)
    for G, kg in ((1, 1), (8, 8), (64, 64)):
        g = router.grouped_topk_softmax(logits, 8, G, kg, True)
        assert np.array_equal(g[0], plain[0]) and np.array_equal(g[1], plain[1])


def test_grouped_invariants_and_group_score_is_the_best_logit():
    rng = np.random.default_rng(9)
    logits = (rng.standard_normal((100, 128)) * 2).astype(np.float32)
    ids, w = router.grouped_topk_softmax(logits, 8, 8, 3, True)
    groups = ids // 16
    assert all(len(set(r)) <= 3 for r in groups.tolist())
    gmax = logits.reshape(100, 8, 16).max(axis=2)
    third = np.sort(gmax, axis=1)[:, ::-1][:, 2]
    for t in range(100):
        assert all(gmax[t, g] >= third[t] for g in set(groups[t].tolist()))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)
    # one strong expert beats two moderate ones: the score is the maximum, not a sum
    l = np.array([[5.0, -9, -9, -9, 3.0, 3.0, -9, -9]], np.float32)
    ids, _ = router.grouped_topk_softmax(l, 2, 2, 1, True)
    assert ids.tolist() == [[0, 1]]
