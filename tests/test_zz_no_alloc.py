"""GPU test of the scratch-free sort-and-pad, moe_align_noalloc, through the
C ABI: on consecutive calls (a large one, then a smaller one, then a large
one over a different expert count, so each call runs on the scratch the
previous call left behind) its layout is bit-identical to moe_align's with a
caller-owned scratch, over the defined prefix: the sorted pair rows, the
block -> expert table and the padded row count."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import align as ref_align
from tests.gpu_util import align_prefix, note, np_

pytestmark = pytest.mark.gpu


def _ids(T, k, E, seed):
    g = torch.Generator().manual_seed(seed)
    # distinct experts per token, skewed toward low ids (a few heavy experts)
    scores = torch.rand((T, E), generator=g) + torch.linspace(0.5, 0.0, E)
    return scores.topk(k, dim=1).indices.to(torch.int32)


@pytest.mark.parametrize("calls", [
    [(8192, 8, 256, 128), (3, 8, 64, 16), (2048, 6, 96, 64)],
    [(1, 1, 1, 16), (16384, 32, 512, 128), (100, 4, 16, 32)],
])
def test_noalloc_matches_moe_align(calls):
    for T, k, E, bm in calls:
        note(f"moe_align_noalloc T={T} k={k} E={E} block_m={bm}")
        ids_cpu = _ids(T, k, E, T + E)
        ids = ids_cpu.cuda()
        s0, e0, n0 = moe.moe_align(ids, E, bm)
        s1, e1, n1 = moe.moe_align_noalloc(ids, E, bm)
        torch.cuda.synchronize()
        gs0, ge0, gn0 = align_prefix(s0, e0, n0, bm)
        gs1, ge1, gn1 = align_prefix(s1, e1, n1, bm)
        assert gn1 == gn0 and np.array_equal(gs1, gs0) and np.array_equal(ge1, ge0)
        rs, re, rn = ref_align.moe_align(ids_cpu.numpy(), E, bm)
        assert gn1 == rn and np.array_equal(gs1, rs) and np.array_equal(ge1, re)
