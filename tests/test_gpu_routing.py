"""GPU parity of the routing variants (moe_topk_softmax_grouped and
moe_fp8_forward_routed through the C ABI) against the oracle.

Grouped top-k: ids bit-exact and weights within 1e-5 relative, including
ties, a token count that leaves waves idle in the last workgroup, and the
DeepSeek-V3 grouping (256 experts in 8 groups, 4 kept, top 8).  The routed
forward: routing ids (global), the sort-and-pad layout over the local
experts, the pair -> row map (-1 exactly for the pairs of absent experts)
and the activation codes are exact targets; the output meets the layer's
bar.  An identity expert map must reproduce moe_fp8_forward bit for bit,
and a map with no local expert must give zeros."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import align as ref_align
from oracle import moe as ref_moe
from oracle import router as ref_router
from synth import make_activations, make_weights
from tests.gpu_util import WEIGHT_RTOL, align_prefix, assert_out_close, note, np_

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,k,G,kg,renorm", [
    (16, 16, 4, 4, 2, True), (33, 256, 8, 8, 4, True), (7, 64, 6, 8, 3, False),
    (5, 32, 2, 32, 2, True), (130, 12, 3, 3, 1, True), (9, 512, 8, 64, 8, True),
    (64, 96, 4, 8, 2, False)])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_grouped_router(T, E, k, G, kg, renorm, kind):
    note(f"grouped router T={T} E={E} k={k} G={G} kg={kg} {kind}")
    rng = np.random.default_rng(T * E + k + G + kg)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        logits = np.round(logits * 2) / 2
    ids, w = moe.moe_topk_softmax_grouped(torch.from_numpy(logits).cuda(), k, G, kg, renorm)
    torch.cuda.synchronize()
    rids, rw = ref_router.grouped_topk_softmax(logits, k, G, kg, renorm)
    assert np.array_equal(np_(ids), rids)
    np.testing.assert_allclose(np_(w), rw, rtol=WEIGHT_RTOL, atol=0)


def _layer(T, H, I, E, k, seed, EL=None, local=None):
    w13, w13s, w2, w2s = make_weights(H, I, E if local is None else EL, seed)
    x, logits = make_activations(H, E, T, seed * 10)
    return x, logits, (w13, w13s, w2, w2s)


def _routed_case(T, H, I, E, k, G, kg, local, seed, what):
    """local: list of the global experts this rank holds (None: all, no map)"""
    EL = E if local is None else len(local)
    x, logits, ws = _layer(T, H, I, E, k, seed, EL, local)
    emap = None
    if local is not None:
        emap = np.full(E, -1, np.int32)
        emap[np.asarray(local)] = np.arange(EL, dtype=np.int32)
    note(f"routed forward {what} T={T} H={H} I={I} E={E} k={k} G={G} kg={kg} EL={EL}")
    wsp = moe.alloc_workspace(T, H, I, E, k)
    out = moe.moe_fp8_forward_routed(
        x.cuda(), logits.cuda(), *[a.cuda() for a in ws], k, True, G, kg,
        None if emap is None else torch.from_numpy(emap).cuda(), workspace=wsp)
    torch.cuda.synchronize()
    ref, info = ref_moe.moe_forward(x.float().numpy(), logits.numpy(), *[a.numpy() for a in ws], k,
                                    True, num_expert_group=G, topk_group=kg, expert_map=emap)
    taps = moe.workspace_taps(wsp, T, H, I, E, k)
    assert np.array_equal(np_(taps["topk_ids"]), info["ids"]), f"{what}: ids"
    np.testing.assert_allclose(np_(taps["topk_weights"]), info["w"], rtol=WEIGHT_RTOL, atol=0)
    local_ids = info["ids"] if emap is None else emap[info["ids"]]
    bm = taps["block_m"]
    gs, ge, gn = align_prefix(taps["sorted_ids"], taps["expert_ids"], taps["ntpp"], bm)
    rs, re, rn = ref_align.moe_align(local_ids, EL, bm)
    assert gn == rn and np.array_equal(gs, rs) and np.array_equal(ge, re), f"{what}: layout"
    pos = np_(taps["pair_pos"])
    absent = local_ids.reshape(-1) < 0
    assert np.all(pos[absent] == -1) and np.all(pos[~absent] >= 0), f"{what}: pair rows"
    assert np.array_equal(gs[pos[~absent]], np.nonzero(~absent)[0]), f"{what}: pair rows invert"
    assert np.array_equal(np_(taps["xq"]), info["xq"]), f"{what}: xq"
    m = assert_out_close(np_(out.float()), ref, what)
    note(f"  absent pairs {absent.mean():.2f}  max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e}")
    return out


@pytest.mark.parametrize("T,H,I,E,k,G,kg,local", [
    (37, 256, 256, 16, 4, 4, 2, None),                 # grouped, decode blocks
    (300, 384, 256, 8, 2, 4, 2, None),                 # grouped, 128-row blocks
    (41, 256, 384, 12, 3, 1, 1, [0, 5, 7, 11]),        # expert map, decode blocks
    (400, 256, 256, 8, 2, 1, 1, [1, 2, 6]),            # expert map, 128-row blocks
    (64, 512, 256, 64, 6, 8, 3, list(range(16, 32))),  # both, one linear rank of four
    (256, 256, 128, 32, 4, 4, 2, list(range(1, 32, 4))),  # both, round-robin placement
    # at most 16 tokens: the one-launch front end (routing, layout, quant)
    (1, 256, 256, 16, 4, 4, 2, None),                  # grouped, one token
    (16, 256, 384, 12, 3, 1, 1, [0, 5, 7, 11]),        # expert map, sixteen tokens
    (5, 512, 256, 64, 6, 8, 3, list(range(16, 32))),   # both
    (16, 256, 256, 512, 8, 1, 1, None),                # 512 experts
])
def test_routed_forward(T, H, I, E, k, G, kg, local):
    _routed_case(T, H, I, E, k, G, kg, local, seed=T + H + I + E + k + G, what="routed")


def test_identity_map_equals_plain_forward_and_absent_map_gives_zeros():
    T, H, I, E, k = 77, 256, 256, 8, 2
    x, logits, ws = _layer(T, H, I, E, k, 31)
    g = [a.cuda() for a in ws]
    xd, ld = x.cuda(), logits.cuda()
    note("routed forward identity map / absent map")
    plain = moe.moe_fp8_forward(xd, ld, *g, k, True)
    ident = moe.moe_fp8_forward_routed(xd, ld, *g, k, True, 1, 1,
                                       torch.arange(E, dtype=torch.int32, device="cuda"))
    none = moe.moe_fp8_forward_routed(xd, ld, *[a[:1].contiguous() for a in g], k, True, 1, 1,
                                      torch.full((E,), -1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), ident.view(torch.int16))
    assert torch.all(none == 0)


def test_dsv3_grouping_on_one_rank_of_eight():
    """DeepSeek-V3 routing shape (256 experts, 8 groups, 4 kept, top 8) with
    the 32 experts of one rank of an 8-way linear placement, H = 7168,
    I = 2048, T = 8192 (128-row blocks).  Routing, layout, pair rows and
    activation codes on every token; the output on sampled tokens."""
    T, H, I, E, k, G, kg = 8192, 7168, 2048, 256, 8, 8, 4
    local = np.arange(64, 96)
    EL = local.size
    note(f"routed forward dsv3 rank T={T} E={E} EL={EL} G={G} kg={kg}")
    w13, w13s, w2, w2s = make_weights(H, I, EL, 2077, "cuda")
    x, logits = make_activations(H, E, T, 2070, "bias", "cuda")
    emap = np.full(E, -1, np.int32)
    emap[local] = np.arange(EL, dtype=np.int32)
    wsp = moe.alloc_workspace(T, H, I, E, k)
    out = moe.moe_fp8_forward_routed(x, logits, w13, w13s, w2, w2s, k, True, G, kg,
                                     torch.from_numpy(emap).cuda(), workspace=wsp)
    torch.cuda.synchronize()
    taps = moe.workspace_taps(wsp, T, H, I, E, k)
    rids, rw = ref_router.grouped_topk_softmax(np_(logits), k, G, kg, True)
    assert np.array_equal(np_(taps["topk_ids"]), rids)
    np.testing.assert_allclose(np_(taps["topk_weights"]), rw, rtol=WEIGHT_RTOL, atol=0)
    local_ids = emap[rids]
    bm = taps["block_m"]
    assert bm == 128
    gs, ge, gn = align_prefix(taps["sorted_ids"], taps["expert_ids"], taps["ntpp"], bm)
    rs, re, rn = ref_align.moe_align(local_ids, EL, bm)
    assert gn == rn and np.array_equal(gs, rs) and np.array_equal(ge, re)
    pos = np_(taps["pair_pos"])
    absent = local_ids.reshape(-1) < 0
    assert np.all(pos[absent] == -1) and np.array_equal(gs[pos[~absent]], np.nonzero(~absent)[0])
    from oracle import quant as ref_quant
    xq, xs = ref_quant.per_token_group_quant(np_(x.float()))
    assert np.array_equal(np_(taps["xq"]), xq) and np.array_equal(np_(taps["xs"]), xs)
    # sampled tokens, at least two of them with a local pair
    has_local = np.nonzero((local_ids >= 0).any(axis=1))[0]
    rng = np.random.default_rng(5)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(has_local, 4, replace=False),
                                    rng.choice(T, 2, replace=False)]))
    ref, _ = ref_moe.moe_forward(np_(x.float()), np_(logits), np_(w13), np_(w13s), np_(w2),
                                 np_(w2s), k, True, tokens=tok, num_expert_group=G,
                                 topk_group=kg, expert_map=emap)
    m = assert_out_close(np_(out.float())[tok], ref, "dsv3 rank")
    note(f"  local pairs {(~absent).mean():.3f}  max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e}")
