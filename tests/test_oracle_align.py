"""Pins of oracle/align.py: numpy's stable argsort, the bijection of the
non-sentinel entries onto [0, P), one expert per block, and block counts."""

import numpy as np
import pytest

from oracle import align


def _check(ids, E, BM):
    sorted_ids, expert_ids, ntpp = align.moe_align(ids, E, BM)
    flat = ids.reshape(-1)
    P = flat.size
    assert ntpp == sorted_ids.size and ntpp % BM == 0
    assert expert_ids.size == ntpp // BM
    real = sorted_ids[sorted_ids != P]
    # stable sort by expert is the concatenation of the non-sentinel entries
    assert np.array_equal(real, np.argsort(flat, kind="stable"))
    # bijection onto [0, P)
    assert np.array_equal(np.sort(real), np.arange(P))
    # each block holds one expert, and the block's real pairs route there
    blocks = sorted_ids.reshape(-1, BM)
    for b in range(blocks.shape[0]):
        r = blocks[b][blocks[b] != P]
        assert r.size > 0 and np.all(flat[r] == expert_ids[b])
    # blocks per expert = ceil(cnt / BM), in expert order
    cnt = np.bincount(flat, minlength=E)
    nb = -(-cnt // BM)
    assert np.array_equal(expert_ids, np.repeat(np.arange(E), nb))
    return sorted_ids, expert_ids, ntpp


@pytest.mark.parametrize("T,E,k,BM", [(16, 8, 2, 16), (64, 256, 8, 16), (33, 128, 8, 32),
                                      (1, 128, 8, 16), (5, 4, 4, 64), (300, 8, 2, 128)])
def test_random_routing(T, E, k, BM):
    rng = np.random.default_rng(T + E + k + BM)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check(ids, E, BM)


def test_worked_layout():
    # pairs p = t*k + j: t0 -> (2, 0), t1 -> (0, 1), t2 -> (2, 1); BM = 2, P = 6
    ids = np.array([[2, 0], [0, 1], [2, 1]], dtype=np.int32)
    s, e, n = _check(ids, 4, 2)
    assert s.tolist() == [1, 2, 3, 5, 0, 4]
    assert e.tolist() == [0, 1, 2] and n == 6
    s, e, n = _check(ids, 4, 4)
    assert s.tolist() == [1, 2, 6, 6, 3, 5, 6, 6, 0, 4, 6, 6] and e.tolist() == [0, 1, 2]


def test_all_to_one_expert_and_empty_experts():
    ids = np.full((37, 1), 3, dtype=np.int32)
    s, e, n = _check(ids, 8, 16)
    assert n == 48 and e.tolist() == [3, 3, 3]
    assert np.all(s[37:] == 37)
