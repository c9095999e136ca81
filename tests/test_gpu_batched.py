"""GPU parity of the batched (masked) expert format (moe_fp8_batched_experts
through the C ABI) against oracle/moe.py's batched_experts.

The sort-and-pad layout built from the device counts, the token -> row map
(-1 past each count) and the activation codes of the real rows are exact
targets; the output meets the layer's bar on the real rows and is exactly
zero past each count.  Counts include empty and full experts; the input rows
past the counts hold NaN, which must never reach the output.  One case
replays the call on the same buffers with new device counts."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import align as ref_align
from oracle import moe as ref_moe
from oracle import quant as ref_quant
from synth import make_weights
from tests.gpu_util import align_prefix, assert_out_close, note, np_

pytestmark = pytest.mark.gpu


def _inputs(E, M, H, counts, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((E, M, H), generator=g).to(torch.bfloat16)
    for e in range(E):
        x[e, counts[e]:] = float("nan")
    return x


def _check(x, counts, w, out, wsp, E, M, H, I, what):
    ref, _ = ref_moe.batched_experts(x.float().numpy(), counts, *[a.numpy() for a in w])
    T = E * M
    taps = moe.workspace_taps(wsp, T, H, I, E, 1)
    ids = np.where(np.arange(M)[None, :] < counts[:, None], np.arange(E)[:, None], -1)
    bm = taps["block_m"]
    gs, ge, gn = align_prefix(taps["sorted_ids"], taps["expert_ids"], taps["ntpp"], bm)
    rs, re, rn = ref_align.moe_align(ids.reshape(-1, 1), E, bm)
    assert gn == rn and np.array_equal(gs, rs) and np.array_equal(ge, re), f"{what}: layout"
    pos = np_(taps["pair_pos"])
    real = ids.reshape(-1) >= 0
    assert np.all(pos[~real] == -1) and np.array_equal(gs[pos[real]], np.nonzero(real)[0])
    xr = x.float().numpy().reshape(T, H)[real]
    xq, xs = ref_quant.per_token_group_quant(xr)
    assert np.array_equal(np_(taps["xq"])[real], xq) and np.array_equal(np_(taps["xs"])[real], xs)
    o = np_(out.float())
    for e in range(E):
        assert np.all(o[e, counts[e]:] == 0), f"{what}: rows past the count of expert {e}"
    m = assert_out_close(o.reshape(T, H)[real], ref.reshape(T, H)[real], what)
    note(f"  block_m={bm} rows={int(real.sum())} max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e}")


@pytest.mark.parametrize("E,M,H,I,counts", [
    (4, 16, 256, 256, [3, 0, 16, 9]),                  # 16-row blocks, an empty and a full expert
    (8, 40, 384, 256, [40, 1, 0, 17, 33, 40, 2, 5]),   # 64-row blocks
    (3, 128, 256, 384, [128, 70, 0]),                  # 128-row blocks
    (2, 300, 512, 256, [299, 300]),                    # 128-row blocks, several per expert
    (1, 64, 256, 128, [0]),                            # nothing to do
])
def test_batched_experts(E, M, H, I, counts):
    counts = np.asarray(counts, np.int32)
    note(f"batched experts E={E} M={M} H={H} I={I} counts={counts.tolist()}")
    x = _inputs(E, M, H, counts, E * M + H)
    w = make_weights(H, I, E, E + M + I)
    wsp = torch.empty(moe.moe_fp8_batched_workspace_bytes(E, M, H, I), dtype=torch.uint8, device="cuda")
    out = moe.moe_fp8_batched_experts(x.cuda(), torch.from_numpy(counts).cuda(),
                                      *[a.cuda() for a in w], workspace=wsp)
    torch.cuda.synchronize()
    _check(x, counts, w, out, wsp, E, M, H, I, "batched")


def test_batched_experts_replay_with_new_counts():
    E, M, H, I = 6, 32, 256, 256
    w = make_weights(H, I, E, 41)
    wd = [a.cuda() for a in w]
    wsp = torch.empty(moe.moe_fp8_batched_workspace_bytes(E, M, H, I), dtype=torch.uint8, device="cuda")
    cnt_dev = torch.zeros(E, dtype=torch.int32, device="cuda")
    x_dev = torch.empty((E, M, H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((E, M, H), dtype=torch.bfloat16, device="cuda")
    for i, counts in enumerate(([5, 0, 32, 7, 1, 12], [0, 31, 2, 0, 16, 32])):
        counts = np.asarray(counts, np.int32)
        note(f"batched replay {i} counts={counts.tolist()}")
        x = _inputs(E, M, H, counts, 100 + i)
        x_dev.copy_(x.cuda())
        cnt_dev.copy_(torch.from_numpy(counts).cuda())
        moe.moe_fp8_batched_experts(x_dev, cnt_dev, *wd, out=out, workspace=wsp)
        torch.cuda.synchronize()
        _check(x, counts, w, out, wsp, E, M, H, I, f"replay {i}")
