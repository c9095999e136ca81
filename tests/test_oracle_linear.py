"""Pins of the dense block-FP8 linear oracle (oracle/linear.py).

* a brute force: the scalar group quantiser, then each output as a sum over
  128-wide K blocks with both scales indexed explicitly
  (xs[m, kb] * w_scale[n // 128, kb]), decoding through torch's float8
  conversion;
* planted mistakes (transposed block-scale indexing, a dropped activation
  scale) fail it;
* a closed form: unit scales and activations on the e4m3 grid with a group
  maximum of 448 make every product exact, so the float64 result is the exact
  integer-grid product;
* permuting the rows of x permutes the output;
* doubling the weight scales doubles the output exactly;
* a loose agreement with the unquantised float64 product.
"""

import math

import numpy as np
import torch

from oracle import linear, quant
from oracle.moe import bf16_round
from synth import block_quantize_e4m3, make_linear, make_mx_linear, mx_quantize_e4m3
from tests import _brute

DEC = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _inputs(M=3, N=384, K=384, seed=11):
    x, w, ws = make_linear(M, N, K, seed)
    return x.float().numpy(), w.numpy(), ws.numpy()


def _brute_force(x, w, ws, transpose_scales=False, drop_act_scale=False):
    M, K = x.shape
    N = w.shape[0]
    xq = np.zeros((M, K), np.uint8)
    xs = np.zeros((M, K // 128), np.float32)
    for m in range(M):
        for g in range(K // 128):
            c, s = _brute.quant_group_scalar(x[m, 128 * g:128 * (g + 1)])
            xq[m, 128 * g:128 * (g + 1)] = c
            xs[m, g] = s
    acc = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            total = 0.0
            for kb in range(K // 128):
                part = float(np.dot(DEC[xq[m, 128 * kb:128 * (kb + 1)]], DEC[w[n, 128 * kb:128 * (kb + 1)]]))
                sw = ws[kb, n // 128] if transpose_scales else ws[n // 128, kb]
                sa = 1.0 if drop_act_scale else float(xs[m, kb])
                total += sa * float(sw) * part
            acc[m, n] = total
    return acc


def test_matches_brute_force():
    x, w, ws = _inputs()
    out, info = linear.block_fp8_linear(x, w, ws)
    ref = _brute_force(x, w, ws)
    np.testing.assert_allclose(info["acc"], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out, bf16_round(ref))


def test_planted_mistakes_fail():
    x, w, ws = _inputs()
    _, info = linear.block_fp8_linear(x, w, ws)
    for kw in ({"transpose_scales": True}, {"drop_act_scale": True}):
        bad = _brute_force(x, w, ws, **kw)
        assert not np.allclose(info["acc"], bad, rtol=1e-3, atol=1e-6), kw


def test_closed_form_unit_scales():
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    M, N, K = 4, 256, 384
    xc = rng.choice(finite, size=(M, K))
    xc[:, ::128] = 0x7E            # each group's maximum is +448, so its scale is exactly 1
    x = DEC[xc].astype(np.float32)
    w = rng.choice(finite, size=(N, K)).astype(np.uint8)
    ws = np.ones((N // 128, K // 128), np.float32)
    out, info = linear.block_fp8_linear(x, w, ws)
    assert np.array_equal(info["xs"], np.ones((M, K // 128), np.float32))
    assert np.array_equal(info["xq"], xc)
    exact = DEC[xc] @ DEC[w].T      # every term and partial sum is exact in float64
    assert np.array_equal(info["acc"], exact)
    assert np.array_equal(out, bf16_round(exact))


def test_row_permutation_and_scale_doubling():
    x, w, ws = _inputs(M=6, N=256, K=256, seed=3)
    out, _ = linear.block_fp8_linear(x, w, ws)
    perm = np.array([4, 1, 5, 0, 3, 2])
    out_p, _ = linear.block_fp8_linear(x[perm], w, ws)
    assert np.array_equal(out_p, out[perm])
    out2, _ = linear.block_fp8_linear(x, w, ws * 2)
    assert np.array_equal(out2, out * 2)


def test_loose_match_to_unquantised_product():
    M, N, K = 5, 256, 512
    g = torch.Generator().manual_seed(9)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    wf = torch.randn((N, K), generator=g) * 0.02
    wq, ws = block_quantize_e4m3(wf)
    out, _ = linear.block_fp8_linear(x.float().numpy(), wq.numpy(), ws.numpy())
    ref = x.double().numpy() @ wf.double().numpy().T
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.08, rel


# ---- MXFP8 ([1, 32] blocks, UE8M0 exponents) ----

def _mx_inputs(M=3, N=256, K=256, seed=13):
    x, w, we = make_mx_linear(M, N, K, seed)
    return x.float().numpy(), w.numpy(), we.numpy()


def _mx_brute_force(x, w, we, block=32, transpose_exponents=False):
    """Scalar brute force: each activation 32-group quantised with a scale
    rounded up to a power of two by exact log2, codes by exhaustive search,
    then every output a sum over 32-wide blocks with both exponents indexed
    explicitly.  With block=128 the activation scale covers 128 columns."""
    M, K = x.shape
    N = w.shape[0]
    acc = np.zeros((M, N))
    xd = np.zeros((M, K))
    for m in range(M):
        for g in range(K // block):
            vals = [np.float32(v) for v in x[m, block * g:block * (g + 1)]]
            amax = max(abs(v) for v in vals)
            s32 = np.float32(max(amax, np.float32(1e-8))) / np.float32(448)
            p = 2.0 ** math.ceil(math.log2(float(s32)))
            for i, v in enumerate(vals):
                xd[m, block * g + i] = DEC[_brute.nearest_code(np.float32(v / np.float32(p)))] * p
    for m in range(M):
        for n in range(N):
            total = 0.0
            for b in range(K // 32):
                e = we[b, n] if transpose_exponents else we[n, b]
                part = float(np.dot(xd[m, 32 * b:32 * (b + 1)], DEC[w[n, 32 * b:32 * (b + 1)]]))
                total += part * 2.0 ** (int(e) - 127)
            acc[m, n] = total
    return acc, xd


def test_mx_matches_brute_force():
    x, w, we = _mx_inputs()
    out, info = linear.mxfp8_linear(x, w, we)
    ref, xd = _mx_brute_force(x, w, we)
    assert np.array_equal(linear.mx_dequant(info["xq"], info["xe"]), xd)
    np.testing.assert_allclose(info["acc"], ref, rtol=1e-12, atol=1e-14)
    assert np.array_equal(out, bf16_round(ref))


def test_mx_planted_mistakes_fail():
    x, w, we = _mx_inputs(N=256, K=256)
    # With power-of-two scales the e4m3 rounding of x / s does not depend on
    # s while x / s stays normal, so a 128-wide scale block shows only where
    # it pushes a group into the subnormal range: make one 32-group tiny.
    x[:, 64:96] *= np.float32(2.0 ** -10)
    _, info = linear.mxfp8_linear(x, w, we)
    _, xd_bad = _mx_brute_force(x, w, we, block=128)
    xd = linear.mx_dequant(info["xq"], info["xe"])
    assert not np.allclose(xd[:, 64:96], xd_bad[:, 64:96], rtol=1e-2, atol=0)
    # 8 weight rows over K = 256 give a square 8 x 8 exponent table, so the
    # transposed indexing stays in range
    w8, we8 = w[:8], we[:8].copy()
    we8[np.triu_indices_from(we8, 1)] += 1           # not symmetric
    _, info = linear.mxfp8_linear(x, w8, we8)
    bad, _ = _mx_brute_force(x, w8, we8, transpose_exponents=True)
    assert not np.allclose(info["acc"], bad, rtol=1e-3, atol=1e-9)


def test_mx_exponent_covariance_and_unit_case():
    x, w, we = _mx_inputs(M=4, N=128, K=256, seed=7)
    out, _ = linear.mxfp8_linear(x, w, we)
    out2, _ = linear.mxfp8_linear(x, w, (we + 1).astype(np.uint8))
    assert np.array_equal(out2, out * 2)
    # unit exponents, activations on the e4m3 grid with a 32-group maximum of
    # 448: every scale is 1 and the product is the exact code product
    rng = np.random.default_rng(6)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    xc = rng.choice(finite, size=(3, 128))
    xc[:, ::32] = 0x7E
    wc = rng.choice(finite, size=(128, 128)).astype(np.uint8)
    out, info = linear.mxfp8_linear(DEC[xc].astype(np.float32), wc, np.full((128, 4), 127, np.uint8))
    assert np.array_equal(info["xe"], np.full((3, 4), 127, np.uint8))
    assert np.array_equal(info["acc"], DEC[xc] @ DEC[wc].T)


def test_mx_loose_match_to_unquantised_product():
    M, N, K = 5, 256, 512
    g = torch.Generator().manual_seed(10)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    wf = torch.randn((N, K), generator=g) * 0.02
    wq, we = mx_quantize_e4m3(wf)
    assert np.all(np.abs(DEC[wq.numpy()]) <= 448)
    out, _ = linear.mxfp8_linear(x.float().numpy(), wq.numpy(), we.numpy())
    ref = x.double().numpy() @ wf.double().numpy().T
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.08, rel
