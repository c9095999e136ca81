"""Sort-and-pad of routed (token, slot) pairs by expert ("moe_align").

Test infrastructure (see the package docstring).

Source: the "Triton Fused MoE Kernel" section of the overview page describes
the sorted-token pattern: every program block takes a BLOCK_SIZE_M chunk of
sorted tokens that all belong to one expert.  The layer definition names the
step "sort and pad tokens by expert" and asks for the layout bit for bit.

Definition (P = T * top_k pairs, pair index p = t * top_k + j):
  cnt[e]   = number of pairs p with ids.flat[p] == e
  pad[e]   = ceil(cnt[e] / BM) * BM            (0 for an expert with no pair)
  off[e]   = sum of pad[e'] for e' < e
  sorted_ids[off[e] + r] = the r-th pair routed to e, in ascending p, r < cnt[e]
  sorted_ids[off[e] + r] = P (the padding sentinel) for cnt[e] <= r < pad[e]
  expert_ids[b]          = e for every BM-row block b inside [off[e], off[e]+pad[e])
  num_tokens_post_padded = sum of pad[e]
Only the prefix [0, num_tokens_post_padded) of sorted_ids and the first
num_tokens_post_padded / BM entries of expert_ids are defined.

Readings: the sentinel is P; empty experts get no block; within an expert the
pairs keep ascending p (a stable sort).

Pinned by tests/test_oracle_align.py (numpy's stable argsort, the bijection
onto [0, P), one expert per block, block counts per expert).
"""

import numpy as np


def moe_align(ids, num_experts: int, block_m: int):
    """ids: int [T, k] expert ids.  Returns (sorted_ids int32 [ntpp],
    expert_ids int32 [ntpp // block_m], ntpp int)."""
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    P = flat.size
    sorted_ids = []
    expert_ids = []
    for e in range(num_experts):
        pairs = [p for p in range(P) if flat[p] == e] if P <= 4096 else \
            list(np.nonzero(flat == e)[0])
        cnt = len(pairs)
        pad = -(-cnt // block_m) * block_m
        sorted_ids.extend(int(p) for p in pairs)
        sorted_ids.extend([P] * (pad - cnt))
        expert_ids.extend([e] * (pad // block_m))
    ntpp = len(sorted_ids)
    return (np.asarray(sorted_ids, dtype=np.int32),
            np.asarray(expert_ids, dtype=np.int32), ntpp)
