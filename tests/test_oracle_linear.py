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

import numpy as np
import torch

from oracle import linear, quant
from oracle.moe import bf16_round
from synth import block_quantize_e4m3, make_linear
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
