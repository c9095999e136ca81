"""GPU parity of the MXFP8 MoE layer (moe_fp8_mx_forward through the C ABI)
against the oracle (oracle/moe.py, moe_forward with mx=True).

Exact targets, read from the workspace taps: routing ids, the sort-and-pad
layout and the group-32 activation codes and UE8M0 bytes of x.
The requantised activation is not an exact target: both GEMMs accumulate on
FP8 MFMAs that apply the exponents in hardware (about 1e-6 of sum |p| on
operands of normal magnitude), so an element next to a rounding midpoint,
or a group maximum next to a power of two, can round the other way.  The
test compares it dequantised: every element within one e4m3 step of the
oracle's (1/8 relative, or one subnormal step of the larger scale, plus
2^-14 of the group's largest value for the accumulation error), and at
most 1% (+3) of the elements differing at all.  The bf16 output meets the
layer's bar on the synthetic MXFP8 weights.  The small cases also run with
the weights' exponents drawn at random around their natural value per block
(weight blocks up to 8x apart), so that an exponent applied to the wrong
block would show as a power of two: there the requantised activation is
checked as above and the output by its relative norm error only, since a
requant code flip times an 8x weight block can move a near-zero output by
more than the elementwise bar allows."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import align as ref_align
from oracle import e4m3
from oracle import moe as ref_moe
from oracle import quant as ref_quant
from oracle import router as ref_router
from synth import make_activations, make_mx_weights
from tests.gpu_util import WEIGHT_RTOL, align_prefix, assert_out_close, note, np_

pytestmark = pytest.mark.gpu


def _deq(q, e):
    return ref_quant.mx_dequant(q, e)


def _compare_mx_requant(g, ge, r, re_):
    """g, r: codes [n, I]; ge, re_: exponent bytes [n, I/32]; returns the
    fraction of elements whose dequantised value differs, and their count"""
    a_g, a_r = _deq(g, ge), _deq(r, re_)
    n, I = g.shape
    step = np.ldexp(1.0, np.repeat(np.maximum(ge, re_).astype(np.int64) - 127 - 9, 32, axis=1))
    # the FP8 MFMAs' accumulation error is absolute (~1e-6 of sum |p|): near-zero
    # values of a group may move by a few subnormal steps, so allow 2^-14 of the
    # group's largest magnitude on top
    gmax = np.repeat(np.abs(a_r).reshape(n, I // 32, 32).max(axis=2), 32, axis=1)
    allowed = 0.125 * np.maximum(np.abs(a_g), np.abs(a_r)) + step + gmax * 2.0 ** -14
    worst = np.max(np.abs(a_g - a_r) - allowed)
    assert worst <= 0, f"a requantised value is {worst} beyond one e4m3 step"
    diff = a_g != a_r
    return float(diff.mean()), diff.size


def _run(x, logits, w, T, H, I, E, k):
    wsp = torch.empty(moe.moe_fp8_mx_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device="cuda")
    out = moe.moe_fp8_mx_forward(x, logits, *w, k, True, workspace=wsp)
    torch.cuda.synchronize()
    return out, moe.workspace_taps(wsp, T, H, I, E, k, mx=True)


def _check_front(taps, x_np, rids, rw, E):
    assert np.array_equal(np_(taps["topk_ids"]), rids), "ids"
    np.testing.assert_allclose(np_(taps["topk_weights"]), rw, rtol=WEIGHT_RTOL, atol=0)
    bm = taps["block_m"]
    gs, ge, gn = align_prefix(taps["sorted_ids"], taps["expert_ids"], taps["ntpp"], bm)
    rs, re_, rn = ref_align.moe_align(rids, E, bm)
    assert gn == rn and np.array_equal(gs, rs) and np.array_equal(ge, re_), "layout"
    xq, _, xe = ref_quant.per_token_group_quant_pow2(x_np, 32)
    assert np.array_equal(np_(taps["xq"]), xq) and np.array_equal(np_(taps["xs"]), xe), "x codes"
    return gs


def _requant_of_pairs(taps, rows, pairs, P):
    inv = np.full(P, -1, np.int64)
    real = rows < P
    inv[rows[real]] = np.nonzero(real)[0]
    pos = torch.from_numpy(inv[pairs]).to(taps["aq"].device)
    return np_(taps["aq"][pos]), np_(taps["as"][pos])


@pytest.mark.parametrize("T,H,I,E,k", [
    (5, 256, 256, 8, 2),       # 16-row blocks
    (37, 256, 384, 4, 4),      # top_k = E, 64-row blocks (four 16-row workgroups), odd K blocks
    (300, 384, 256, 2, 1),     # 128-row blocks, several per expert
    (64, 512, 512, 16, 3),     # 32-row blocks, exponents in 16-byte groups (K % 512 == 0)
    (64, 512, 1024, 4, 2),     # 64-row blocks on the 16-byte exponent groups, 8 K blocks in GEMM2
    (40, 1024, 640, 8, 2),     # grouped exponents in GEMM1, per-block bytes in GEMM2 (5 K blocks)
    (20, 256, 256, 64, 6),     # many small experts, heavy padding
    (4096, 2048, 256, 4, 2),   # 128-row blocks, 544 GEMM2 tiles: several per persistent workgroup
])
@pytest.mark.parametrize("spread", [False, True])
def test_mx_small_layers(T, H, I, E, k, spread):
    note(f"mx forward T={T} H={H} I={I} E={E} k={k} spread={spread}")
    seed = T + H + I + E + k
    w13, w13e, w2, w2e = make_mx_weights(H, I, E, seed)
    if spread:
        g = torch.Generator().manual_seed(seed + 1)
        w13e = (w13e.int() + torch.randint(-3, 4, w13e.shape, generator=g)).to(torch.uint8)
        w2e = (w2e.int() + torch.randint(-3, 4, w2e.shape, generator=g)).to(torch.uint8)
    x, logits = make_activations(H, E, T, seed * 10)
    w = [a.cuda() for a in (w13, w13e, w2, w2e)]
    out, taps = _run(x.cuda(), logits.cuda(), w, T, H, I, E, k)
    ref, info = ref_moe.moe_forward(x.float().numpy(), logits.numpy(), w13.numpy(), w13e.numpy(),
                                    w2.numpy(), w2e.numpy(), k, True, mx=True)
    rows = _check_front(taps, x.float().numpy(), info["ids"], info["w"], E)
    g, ge = _requant_of_pairs(taps, rows, np.arange(T * k), T * k)
    mm, n = _compare_mx_requant(g, ge, info["aq"], info["as"])
    assert mm * n <= 0.01 * n + 3, f"requant mismatch fraction {mm}"
    o = np_(out.float())
    if spread:
        assert np.isfinite(o).all()
        rel = float(np.linalg.norm(o - ref) / np.linalg.norm(ref))
        assert rel < 1e-2, f"relative norm error {rel}"
        note(f"  rel_norm={rel:.3e} requant_differing={mm:.2e}")
    else:
        m = assert_out_close(o, ref, "mx small")
        note(f"  max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e} requant_differing={mm:.2e}")


def _misaligned_copy(t):
    """t's bytes at an address 4 bytes past a 16-byte boundary (the C ABI
    asks 4-byte alignment of the exponent arrays)"""
    buf = torch.empty(t.numel() + 16, dtype=torch.uint8, device="cuda")
    base = (-buf.data_ptr()) % 16
    v = buf[base + 4:base + 4 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == 4
    return v


@pytest.mark.parametrize("T,H,I,E,k", [(6, 512, 512, 8, 2), (64, 512, 1024, 4, 2)])
def test_mx_misaligned_exponents_match(T, H, I, E, k):
    """With K a multiple of 512 the decode GEMMs read the weight exponents in
    aligned 16-byte groups; exponent arrays that are only 4-byte aligned take
    the per-block byte loads instead.  Both apply the same exponents to the
    same MFMAs, so the requantised activation and the output are identical."""
    note(f"mx forward misaligned exponents T={T} H={H} I={I} E={E} k={k}")
    w13, w13e, w2, w2e = (a.cuda() for a in make_mx_weights(H, I, E, 31 + T))
    x, logits = (a.cuda() for a in make_activations(H, E, T, 310 + T))
    out_a, taps_a = _run(x, logits, [w13, w13e, w2, w2e], T, H, I, E, k)
    out_b, taps_b = _run(x, logits, [w13, _misaligned_copy(w13e), w2, _misaligned_copy(w2e)],
                         T, H, I, E, k)
    assert taps_a["block_m"] <= 64, "decode-sized blocks expected"
    # the rows of real pairs (padding rows are never written)
    bm, P = taps_a["block_m"], T * k
    rows, _, _ = align_prefix(taps_a["sorted_ids"], taps_a["expert_ids"], taps_a["ntpp"], bm)
    ga, gea = _requant_of_pairs(taps_a, rows, np.arange(P), P)
    gb, geb = _requant_of_pairs(taps_b, rows, np.arange(P), P)
    assert np.array_equal(ga, gb) and np.array_equal(gea, geb), "requantised rows differ"
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "outputs differ"


@pytest.mark.parametrize("T", [64, 8192])
def test_mx_full_size_dsv3(T):
    """DeepSeek-V3 shape (H 7168, I 2048, 256 experts, top 8) with MXFP8
    weights; routing, layout and x codes on every token, the requantised
    rows and the output on sampled tokens."""
    H, I, E, k = 7168, 2048, 256, 8
    note(f"mx forward full-size dsv3 T={T}")
    w = make_mx_weights(H, I, E, 2002, "cuda")
    x, logits = make_activations(H, E, T, 2000, "bias", "cuda")
    out, taps = _run(x, logits, w, T, H, I, E, k)
    logits_np, x_np = np_(logits), np_(x.float())
    rids, rw = ref_router.topk_softmax(logits_np, k, True)
    rows = _check_front(taps, x_np, rids, rw, E)
    tok = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(T + 7).choice(T, min(T, 4), replace=False)]))
    experts = np.unique(rids[tok])
    sel = torch.from_numpy(experts).cuda()
    full = []
    for a in w:
        z = np.zeros(tuple(a.shape), np.uint8)
        z[experts] = np_(a[sel])
        full.append(z)
    ref, rinfo = ref_moe.moe_forward(x_np, logits_np, *full, k, True, tokens=tok, mx=True)
    pairs = (tok[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    g, ge = _requant_of_pairs(taps, rows, pairs, T * k)
    mm, n = _compare_mx_requant(g, ge, rinfo["aq"], rinfo["as"])
    assert mm * n <= 0.01 * n + 3, f"requant mismatch fraction {mm}"
    m = assert_out_close(np_(out.float())[tok], ref, f"mx dsv3 T={T}")
    note(f"  sampled {tok.size} tokens: max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e} "
         f"requant_differing={mm:.2e} of {n}")
