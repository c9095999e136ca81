"""Pins of the whole-layer oracle (oracle/moe.py).

* a brute force with explicit loops: routing by full sort, quantisation with
  the exhaustive-search encoder, and each GEMM written per 128-wide K block
  with the block scales indexed explicitly (w_scale[e, n // 128, kb]),
  decoding through torch's float8 conversion;
* E = 1, k = 1 equals a dense gated MLP written as three dense matmuls;
* permuting the tokens permutes the output;
* out(renormalized) = out(raw softmax weights) / sum of the selected
  probabilities, up to bf16 rounding;
* a loose agreement with the unquantized float64 MLP on the same weights;
* planted mistakes in the oracle fail the brute-force pin.
"""

import numpy as np
import pytest
import torch
from scipy.special import softmax

from oracle import moe, quant, router
from synth import make_activations, make_weights, moe_workload
from tests import _brute

DEC = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _layer(T=3, H=256, I=256, E=4, k=2, seed=7, logits_kind="normal"):
    w13, w13s, w2, w2s = make_weights(H, I, E, seed)
    x, logits = make_activations(H, E, T, seed * 10, logits_kind)
    return (x.float().numpy(), logits.numpy(), w13.numpy(), w13s.numpy(),
            w2.numpy(), w2s.numpy())


def _quant_row(row):
    codes, scales = [], []
    for g in range(len(row) // 128):
        c, s = _brute.quant_group_scalar(row[128 * g:128 * (g + 1)])
        codes += c
        scales.append(s)
    return np.array(codes, np.uint8), np.array(scales, np.float32)


def _blocked_matvec(wq, ws, v):
    """out[n] = sum_kb ws[n//128, kb] * sum_{kk in kb} dec(wq[n, kk]) * v[kk]"""
    N, K = wq.shape
    out = np.zeros(N)
    for n in range(N):
        acc = 0.0
        for kb in range(K // 128):
            seg = slice(128 * kb, 128 * kb + 128)
            acc += float(ws[n // 128, kb]) * float(np.dot(DEC[wq[n, seg]], v[seg]))
        out[n] = acc
    return out


def brute_layer(x, logits, w13, w13s, w2, w2s, k, renorm):
    T, H = x.shape
    E = logits.shape[1]
    I = w2.shape[2]
    out = np.zeros((T, H), np.float32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        p = softmax(logits[t].astype(np.float64))[order]
        wts = (p / p.sum() if renorm else p).astype(np.float32)
        xq, xs = _quant_row(x[t])
        xhat = DEC[xq] * np.repeat(xs.astype(np.float64), 128)
        acc = np.zeros(H)
        for j, e in enumerate(order):
            h = _blocked_matvec(w13[e], w13s[e], xhat)
            g, u = h[:I], h[I:]
            a = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
            aq, as_ = _quant_row(a)
            ahat = DEC[aq] * np.repeat(as_.astype(np.float64), 128)
            y = _blocked_matvec(w2[e], w2s[e], ahat)
            acc += float(wts[j]) * y
        out[t] = torch.from_numpy(acc).to(torch.bfloat16).to(torch.float32).numpy()
    return out


def _assert_close_bf16(a, b, exact_frac=0.99):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    np.testing.assert_allclose(a, b, rtol=2.0 ** -7, atol=1e-6)
    assert np.mean(a == b) >= exact_frac


@pytest.mark.parametrize("renorm", [True, False])
def test_brute_force_layer(renorm):
    x, logits, w13, w13s, w2, w2s = _layer()
    out, info = moe.moe_forward(x, logits, w13, w13s, w2, w2s, 2, renorm)
    ref = brute_layer(x, logits, w13, w13s, w2, w2s, 2, renorm)
    _assert_close_bf16(out, ref)


def test_single_expert_is_dense_gated_mlp():
    x, logits, w13, w13s, w2, w2s = _layer(T=5, E=1, I=384)
    out, _ = moe.moe_forward(x, logits, w13, w13s, w2, w2s, 1, True)
    I = w2.shape[2]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    kron = lambda s: np.kron(s.astype(np.float64), np.ones((128, 128)))
    W1 = DEC[w13[0, :I]] * kron(w13s[0, :I // 128])
    W3 = DEC[w13[0, I:]] * kron(w13s[0, I // 128:])
    W2 = DEC[w2[0]] * kron(w2s[0])
    rows = []
    for r in range(x.shape[0]):
        q, s = _quant_row(x[r])
        rows.append(DEC[q] * np.repeat(s.astype(np.float64), 128))
    X = t(np.stack(rows))
    g = X @ t(W1).T
    u = X @ t(W3).T
    A = (torch.nn.functional.silu(g) * u).to(torch.float32).numpy()
    Ahat = np.stack([DEC[q] * np.repeat(s.astype(np.float64), 128)
                     for q, s in map(_quant_row, A)])
    Y = (t(Ahat) @ t(W2).T).to(torch.bfloat16).to(torch.float32).numpy()
    _assert_close_bf16(out, Y)


def test_token_permutation_equivariance():
    x, logits, w13, w13s, w2, w2s = _layer(T=24, H=256, I=256, E=8, k=2, seed=3)
    out, _ = moe.moe_forward(x, logits, w13, w13s, w2, w2s, 2, True)
    perm = np.random.default_rng(0).permutation(24)
    outp, _ = moe.moe_forward(x[perm], logits[perm], w13, w13s, w2, w2s, 2, True)
    _assert_close_bf16(outp, out[perm], exact_frac=0.999)
    # the token-subset mode gives the same rows as the full forward
    sub, _ = moe.moe_forward(x, logits, w13, w13s, w2, w2s, 2, True, tokens=[5, 0, 17])
    _assert_close_bf16(sub, out[[5, 0, 17]], exact_frac=0.999)


def test_renormalisation_identity():
    x, logits, w13, w13s, w2, w2s = _layer(T=16, E=8, k=3, seed=4)
    on, _ = moe.moe_forward(x, logits, w13, w13s, w2, w2s, 3, True)
    off, _ = moe.moe_forward(x, logits, w13, w13s, w2, w2s, 3, False)
    ids, w_raw = router.topk_softmax(logits, 3, False)
    S = w_raw.astype(np.float64).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(on, off / S, rtol=2.0 ** -7, atol=1e-6)


def test_close_to_unquantized_mlp():
    x, logits, w13, w13s, w2, w2s = _layer(T=16, H=512, I=512, E=4, k=2, seed=9)
    out, info = moe.moe_forward(x, logits, w13, w13s, w2, w2s, 2, True)
    ids, w = info["ids"], info["w"]
    I = w2.shape[2]
    ref = np.zeros_like(out, dtype=np.float64)
    for e in range(4):
        W13 = quant.block_dequant(w13[e], w13s[e])
        W2 = quant.block_dequant(w2[e], w2s[e])
        h = x.astype(np.float64) @ W13.T
        y = (moe.silu(h[:, :I]) * h[:, I:]) @ W2.T
        for j in range(2):
            m = ids[:, j] == e
            ref[m] += w[m, j:j + 1] * y[m]
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.05, rel


def test_bf16_round():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -30, -2.5], np.float64)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    ref[3] = 1.0 + 2 ** -7                        # above the tie: rounds up
    assert moe.bf16_round(v).tolist() == ref.tolist()


def _swap_gate_up(x_rows, w13_e, w13s_e, w2_e, w2s_e):
    I = w2_e.shape[1]
    return moe_real_ffn(x_rows, np.concatenate([w13_e[I:], w13_e[:I]]),
                        np.concatenate([w13s_e[I // 128:], w13s_e[:I // 128]]), w2_e, w2s_e)


moe_real_ffn = moe.expert_ffn


@pytest.mark.parametrize("mutant", ["swap_gate_up", "no_router_weight",
                                    "transposed_block_scales", "inverted_act_scale"])
def test_planted_mistakes_fail_brute_force(mutant, monkeypatch):
    if mutant == "swap_gate_up":
        monkeypatch.setattr(moe, "expert_ffn", _swap_gate_up)
    elif mutant == "no_router_weight":
        real = router.topk_softmax
        monkeypatch.setattr(router, "topk_softmax",
                            lambda l, k, r: (real(l, k, r)[0], np.ones((l.shape[0], k), np.float32)))
    elif mutant == "transposed_block_scales":
        real_bd = quant.block_dequant
        monkeypatch.setattr(quant, "block_dequant",
                            lambda w, ws, block=128: real_bd(w, np.ascontiguousarray(ws[::-1, ::-1]), block))
    else:
        real_q = quant.per_token_group_quant
        def inv(x, group=128):
            q, s = real_q(x, group)
            return q, (np.float32(1.0) / s).astype(np.float32)
        monkeypatch.setattr(quant, "per_token_group_quant", inv)
    with pytest.raises(AssertionError):
        test_brute_force_layer(True)


# ---- expert map (one rank's share of the experts) ----

def _acc(info, top_k):
    w = info["w"].astype(np.float64)
    return sum(w[:, j:j + 1] * info["y"][j::top_k] for j in range(top_k))


def test_expert_map_splits_the_layer_into_rank_shares():
    H, I, E, k, T = 256, 256, 6, 2, 9
    x, logits = make_activations(H, E, T, seed_base=901)
    w13, w13s, w2, w2s = make_weights(H, I, E, 902)
    xf, lf = x.float().numpy(), logits.numpy()
    ws = [a.numpy() for a in (w13, w13s, w2, w2s)]
    full, finfo = moe.moe_forward(xf, lf, *ws, k, True)
    ident, _ = moe.moe_forward(xf, lf, *ws, k, True, expert_map=np.arange(E))
    assert np.array_equal(ident, full)
    total = np.zeros((T, H))
    for local in ([0, 2, 5], [1, 3, 4]):      # two ranks, interleaved placement
        emap = np.full(E, -1)
        emap[local] = np.arange(len(local))
        sub = [a[local] for a in ws]
        out, info = moe.moe_forward(xf, lf, *sub, k, True, expert_map=emap)
        assert np.array_equal(info["ids"], finfo["ids"])
        absent = emap[info["ids"].reshape(-1)] < 0
        assert np.all(info["y"][absent] == 0)
        total += _acc(info, k)
    np.testing.assert_allclose(total, _acc(finfo, k), rtol=1e-12, atol=1e-12)
    none, _ = moe.moe_forward(xf, lf, *[a[:1] for a in ws], k, True, expert_map=np.full(E, -1))
    assert np.all(none == 0)


# ---- batched activation format ----

def test_batched_experts_dispatch_then_combine_equals_the_layer():
    """Dispatch a routed layer into the batched format (expert e's rows are
    its pairs' tokens in ascending pair order), run the batched experts, and
    combine with the routing weights: the float64 sum equals the standard
    forward's before rounding, and the rows past each count are zero."""
    H, I, E, k, T = 256, 256, 5, 2, 13
    x, logits = make_activations(H, E, T, seed_base=911)
    w13, w13s, w2, w2s = make_weights(H, I, E, 912)
    xf, lf = x.float().numpy(), logits.numpy()
    ws = [a.numpy() for a in (w13, w13s, w2, w2s)]
    full, finfo = moe.moe_forward(xf, lf, *ws, k, True)
    flat = finfo["ids"].reshape(-1)
    M = 9
    xb = np.full((E, M, H), np.nan, np.float32)          # rows past the counts are never read
    counts = np.zeros(E, np.int64)
    slot = {}
    for p in range(T * k):
        e = int(flat[p])
        slot[p] = (e, counts[e])
        xb[e, counts[e]] = xf[p // k]
        counts[e] += 1
    assert counts.max() <= M
    out, binfo = moe.batched_experts(xb, counts, *ws)
    acc = np.zeros((T, H))
    for p, (e, r) in slot.items():
        acc[p // k] += float(finfo["w"].reshape(-1)[p]) * binfo["y"][e][r]
    np.testing.assert_allclose(acc, _acc(finfo, k), rtol=1e-12, atol=1e-12)
    for e in range(E):
        assert np.all(out[e, counts[e]:] == 0)
        assert np.array_equal(out[e, :counts[e]], moe.bf16_round(binfo["y"][e]))


def test_batched_experts_rows_are_independent():
    H, I, E, M = 256, 128, 3, 6
    g = torch.Generator().manual_seed(5)
    xb = torch.randn((E, M, H), generator=g).to(torch.bfloat16).float().numpy()
    w13, w13s, w2, w2s = make_weights(H, I, E, 913)
    ws = [a.numpy() for a in (w13, w13s, w2, w2s)]
    counts = np.array([6, 0, 4])
    out, _ = moe.batched_experts(xb, counts, *ws)
    assert np.all(out[1] == 0)
    perm = np.array([3, 1, 0, 2])
    xp = xb.copy()
    xp[2, :4] = xb[2, perm]
    outp, _ = moe.batched_experts(xp, counts, *ws)
    assert np.array_equal(outp[2, :4], out[2, perm])
    assert np.array_equal(outp[0], out[0])


# ---- MXFP8 layer ([1, 32] blocks, power-of-two scales) ----

def _mx_brute_quant(rows):
    """Scalar reference of the group-32 power-of-two quantiser: float64
    dequantised values (exact log2 for the scale, exhaustive nearest code)."""
    import math
    out = np.zeros(rows.shape)
    for r in range(rows.shape[0]):
        for g in range(rows.shape[1] // 32):
            vals = [np.float32(v) for v in rows[r, 32 * g:32 * (g + 1)]]
            amax = max(abs(v) for v in vals)
            s32 = np.float32(max(amax, np.float32(1e-8))) / np.float32(448)
            p = 2.0 ** math.ceil(math.log2(float(s32)))
            for i, v in enumerate(vals):
                c = _brute.nearest_code(np.float32(v / np.float32(p)))
                out[r, 32 * g + i] = float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).double()) * p
    return out


def _mx_weights_torch(q, e):
    """float64 weights from codes and UE8M0 bytes through torch's float8 cast."""
    d = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double()
    ex = torch.from_numpy(np.asarray(e, np.int64) - 127).repeat_interleave(32, dim=1)
    return torch.ldexp(d, ex).numpy()


def test_mx_single_expert_is_a_brute_force_gated_mlp():
    from synth import make_mx_weights
    H, I, T = 128, 128, 3
    x, logits = make_activations(H, 1, T, seed_base=931)
    w13, w13e, w2, w2e = [a.numpy() for a in make_mx_weights(H, I, 1, 932)]
    out, info = moe.moe_forward(x.float().numpy(), logits.numpy(), w13, w13e, w2, w2e, 1, True,
                                mx=True)
    xf = _mx_brute_quant(x.float().numpy())
    h = xf @ _mx_weights_torch(w13[0], w13e[0]).T
    a = (h[:, :I] / (1.0 + np.exp(-h[:, :I])) * h[:, I:]).astype(np.float32)
    y = _mx_brute_quant(a) @ _mx_weights_torch(w2[0], w2e[0]).T
    np.testing.assert_allclose(info["a"], a, rtol=1e-6, atol=0)
    np.testing.assert_allclose(info["y"], y, rtol=1e-9, atol=1e-12)
    assert np.array_equal(out, moe.bf16_round(y))


def test_mx_layer_loosely_matches_the_unquantised_mlp():
    from synth import WEIGHT_STD, mx_quantize_e4m3
    H, I, E, k, T = 256, 256, 4, 2, 8
    x, logits = make_activations(H, E, T, seed_base=941)
    g = torch.Generator().manual_seed(942)
    wf13 = torch.randn((E, 2 * I, H), generator=g) * WEIGHT_STD
    wf2 = torch.randn((E, H, I), generator=g) * WEIGHT_STD
    q = [mx_quantize_e4m3(wf13[e]) for e in range(E)]
    r = [mx_quantize_e4m3(wf2[e]) for e in range(E)]
    w13 = np.stack([a.numpy() for a, _ in q]); w13e = np.stack([b.numpy() for _, b in q])
    w2 = np.stack([a.numpy() for a, _ in r]); w2e = np.stack([b.numpy() for _, b in r])
    out, info = moe.moe_forward(x.float().numpy(), logits.numpy(), w13, w13e, w2, w2e, k, True,
                                mx=True)
    xd = x.double().numpy()
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(info["ids"][t, j])
            h = wf13[e].double().numpy() @ xd[t]
            a = h[:I] / (1 + np.exp(-h[:I])) * h[I:]
            ref[t] += float(info["w"][t, j]) * (wf2[e].double().numpy() @ a)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.1, rel


def test_finish_from_requant_is_the_forward_tail():
    """Steps 7-8 from given requantised codes: fed the forward's own codes it
    reproduces the forward's output bit for bit; fed the codes of a different
    pair for one pair, that pair's token changes and no other token does."""
    w = moe_workload("tiny", 16)
    x, lg = w["x"].float().numpy(), w["logits"].numpy()
    args = (w["w13"].numpy(), w["w13_scale"].numpy(), w["w2"].numpy(), w["w2_scale"].numpy())
    k = w["top_k"]
    out, info = moe.moe_forward(x, lg, *args, k, True)
    again = moe.finish_from_requant(info["aq"], info["as"], info["ids"], info["w"], args[2],
                                        args[3], k)
    assert np.array_equal(again.view(np.uint32), out.view(np.uint32))
    aq = info["aq"].copy()
    aq[5] = info["aq"][9]                          # pair 5 (token 2) takes pair 9's codes
    other = moe.finish_from_requant(aq, info["as"], info["ids"], info["w"], args[2], args[3], k)
    changed = np.nonzero(np.any(other != out, axis=1))[0]
    assert changed.tolist() == [5 // k]
