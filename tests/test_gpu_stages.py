"""GPU parity of the stage entry points against the oracle: the standalone
activation quantiser (codes and scales bit-exact), the router (ids
bit-exact, weights within 1e-5 relative) and the sort-and-pad layout
(bit-exact prefix).  All calls go through the C ABI."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import align as ref_align
from oracle import quant as ref_quant
from oracle import router as ref_router
from synth import QUANT_WORKLOAD, quant_input
from tests.gpu_util import WEIGHT_RTOL, align_prefix, note, np_

pytestmark = pytest.mark.gpu


def _quant_check(x_bf16, rows=None):
    q, s = moe.per_token_group_quant_fp8(x_bf16.cuda())
    torch.cuda.synchronize()
    xf = x_bf16.float().numpy()
    qg, sg = np_(q), np_(s)
    if rows is not None:
        xf, qg, sg = xf[rows], qg[rows], sg[rows]
    rq, rs = ref_quant.per_token_group_quant(xf)
    assert np.array_equal(sg.view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = np.nonzero(qg != rq)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}"


@pytest.mark.parametrize("M,K", [(1, 128), (37, 384), (300, 7168), (5, 2048)])
def test_quant_random_with_outliers(M, K):
    note(f"quant M={M} K={K}")
    _quant_check(quant_input(M, K, seed_base=M * 7 + K))


def test_quant_every_bf16_value():
    # groups whose amax is 448 have scale exactly 1, so every bf16 value in
    # [-448, 448] reaches the e4m3 rounding unchanged
    note("quant every bf16 value")
    b = (np.arange(0, 1 << 16, dtype=np.uint32) << 16).view(np.float32)
    b = b[np.isfinite(b) & (np.abs(b) <= 448.0)]
    b = np.concatenate([b, np.zeros((-b.size) % 127, np.float32)]).reshape(-1, 127)
    x = np.concatenate([np.full((b.shape[0], 1), 448.0, np.float32), b], axis=1)
    _quant_check(torch.from_numpy(x).to(torch.bfloat16))


def test_quant_special_groups():
    note("quant special groups")
    x = np.zeros((6, 256), np.float32)
    x[1, :128] = -0.0                     # negative zeros keep their sign
    x[2, :] = 1e-30                       # below the amax clamp
    x[2, 5] = -1e-30
    x[3, :] = np.float32(2.0 ** -130)     # bf16 subnormals
    x[4, :] = 3.0                         # all equal -> all 448
    x[5, 0] = 1e4
    x[5, 1:] = 1.0                        # an outlier squashes the rest
    x[5, 128:] = -np.arange(128, dtype=np.float32) * 0.37
    _quant_check(torch.from_numpy(x).to(torch.bfloat16))


def test_quant_zero_rows_is_a_no_op():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = moe.per_token_group_quant_fp8(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)


def test_quant_full_size_workload():
    """bf16 [16384, 7168] with 1% outliers, in the launch configuration the
    benchmark times; codes and scales bit-exact on 1024 sampled rows plus the
    first and last."""
    M, K = QUANT_WORKLOAD["M"], QUANT_WORKLOAD["K"]
    note(f"quant full size {M}x{K}")
    x = quant_input(device="cuda")
    q, s = moe.per_token_group_quant_fp8(x)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(0).choice(M, 1024, replace=False)]))
    xr = x[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    rq, rs = ref_quant.per_token_group_quant(xr)
    assert np.array_equal(np_(s)[rows].view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(np_(q)[rows], rq)


FMTS = [(g, f) for g in (32, 128) for f in ("float32", "float32_ceil_ue8m0", "ue8m0")]


def _quant_fmt_check(x_bf16, group, fmt, rows=None):
    q, s = moe.per_token_group_quant_fp8_fmt(x_bf16.cuda(), group, fmt)
    torch.cuda.synchronize()
    xf = x_bf16.float().cpu().numpy()
    qg, sg = np_(q), np_(s)
    if rows is not None:
        xf, qg, sg = xf[rows], qg[rows], sg[rows]
    if fmt == "float32":
        rq, rs = ref_quant.per_token_group_quant(xf, group)
    else:
        rq, rs, rex = ref_quant.per_token_group_quant_pow2(xf, group)
        if fmt == "ue8m0":
            rs = rex
    assert sg.dtype == rs.dtype and np.array_equal(sg.view(np.uint8), rs.view(np.uint8)), "scales differ"
    bad = np.nonzero(qg != rq)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}"


@pytest.mark.parametrize("group,fmt,M,K", [
    (g, f, M, K) for g, f in FMTS
    for M, K in [(1, 128), (37, 384), (301, 7168), (3, 32 * 7 + 96)] if K % g == 0])
def test_quant_fmt_random_with_outliers(group, fmt, M, K):
    note(f"quant fmt={fmt} group={group} M={M} K={K}")
    _quant_fmt_check(quant_input(M, K, seed_base=M * 11 + K + group), group, fmt)


@pytest.mark.parametrize("group,fmt", FMTS)
def test_quant_fmt_special_groups(group, fmt):
    """Scales at and beside exact powers of two (amax = 448 * 2^k, one bf16
    step either side), negative zeros, values under the amax clamp, bf16
    subnormals and the largest bf16 magnitudes."""
    note(f"quant fmt={fmt} group={group} special groups")
    rows = []
    for k in range(-20, 21, 5):
        for step in (-1, 0, 1):
            bits = np.array([448.0 * 2.0 ** k], np.float32).view(np.uint32).astype(np.int64) + (step << 16)
            a = bits.astype(np.uint32).view(np.float32)[0]
            r = np.random.default_rng(100 + k * 3 + step).uniform(-a, a, 2 * group).astype(np.float32)
            r[0], r[group + 1] = a, -a
            rows.append(r)
    x = np.stack(rows)
    z = np.zeros((5, 2 * group), np.float32)
    z[0, :group] = -0.0
    z[1] = 1e-30
    z[2] = np.float32(2.0 ** -130)
    z[3] = 3.0e38
    z[3, 1::2] = -1.5
    z[4, 0] = 1e4
    z[4, 1:] = 1.0
    x = np.concatenate([x, z])
    _quant_fmt_check(torch.from_numpy(x).to(torch.bfloat16), group, fmt)


@pytest.mark.parametrize("group,fmt", [(32, "ue8m0"), (128, "float32_ceil_ue8m0")])
def test_quant_fmt_full_size_workload(group, fmt):
    """bf16 [16384, 7168] with 1% outliers in the launch configuration the
    benchmark times; codes and scales bit-exact on 1024 sampled rows plus the
    first and last."""
    M = QUANT_WORKLOAD["M"]
    note(f"quant fmt={fmt} group={group} full size")
    x = quant_input(device="cuda")
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).choice(M, 1024, replace=False)]))
    _quant_fmt_check(x, group, fmt, rows=rows)


@pytest.mark.parametrize("T,E,k,renorm,kind", [
    (16, 8, 2, True, "normal"), (64, 256, 8, True, "bias"), (33, 128, 8, False, "normal"),
    (1, 128, 8, True, "normal"), (7, 5, 5, True, "normal"), (3, 1, 1, False, "normal"),
    (8192, 256, 8, True, "bias"), (100, 512, 32, True, "normal"), (50, 60, 3, False, "ties"),
    (64, 256, 32, True, "coarse"), (16, 512, 16, False, "equal"), (8, 128, 8, True, "signed_zero")])
def test_router(T, E, k, renorm, kind):
    """The selection's (value, index) order decides every tie: equal logits
    in lanes of different 16-lane rows and register slots ("coarse": seven
    distinct values over 256 experts; "equal": all logits equal, so the ids
    are 0 .. k-1; "signed_zero": -0 and +0, which compare equal)."""
    note(f"router T={T} E={E} k={k} renorm={renorm} {kind}")
    g = torch.Generator().manual_seed(T * 1000 + E + k)
    logits = torch.randn((T, E), generator=g)
    if kind == "bias":
        logits += 0.5 * (torch.randint(0, 2, (E,), generator=g) * 2 - 1)
    if kind == "ties":
        logits = torch.round(logits * 2) / 2       # many equal logits
    if kind == "coarse":
        logits = torch.round(logits).clamp(-3, 3)
    if kind == "equal":
        logits = torch.full((T, E), 0.25)
    if kind == "signed_zero":
        logits = torch.where(torch.rand((T, E), generator=g) < 0.5, torch.tensor(-0.0), torch.tensor(0.0))
    ids, w = moe.moe_topk_softmax(logits.cuda(), k, renorm)
    torch.cuda.synchronize()
    rids, rw = ref_router.topk_softmax(logits.numpy(), k, renorm)
    assert np.array_equal(np_(ids), rids)
    np.testing.assert_allclose(np_(w), rw, rtol=WEIGHT_RTOL, atol=0)


@pytest.mark.parametrize("T,E,k,bm,pattern", [
    (16, 8, 2, 16, "random"), (64, 256, 8, 16, "random"), (1, 128, 8, 16, "random"),
    (512, 8, 2, 128, "random"), (8192, 256, 8, 128, "skew"), (4096, 128, 8, 128, "random"),
    (1000, 64, 4, 32, "one_expert_heavy"), (2048, 16, 1, 64, "all_one"), (129, 512, 8, 256, "random")])
def test_align(T, E, k, bm, pattern):
    note(f"align T={T} E={E} k={k} bm={bm} {pattern}")
    rng = np.random.default_rng(T + E + k + bm)
    if pattern == "all_one":
        ids = np.full((T, k), 3, np.int32)
    else:
        p = np.ones(E)
        if pattern == "skew":
            p = np.exp(rng.standard_normal(E))
        if pattern == "one_expert_heavy":
            p[E // 2] = 50 * E
        p /= p.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    s, e, n = moe.moe_align(torch.from_numpy(ids).cuda(), E, bm)
    torch.cuda.synchronize()
    gs, ge, gn = align_prefix(s, e, n, bm)
    rs, re, rn = ref_align.moe_align(ids, E, bm)
    assert gn == rn
    assert np.array_equal(gs, rs)
    assert np.array_equal(ge, re)
