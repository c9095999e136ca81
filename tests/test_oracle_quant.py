"""Pins of oracle/quant.py: a scalar float32 brute force with the
exhaustive-search encoder, invariants of the scale and codes, the dequant
error bound, special groups, and torch's cast on every bf16 value."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3, quant
from tests import _brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_values(rng, shape, scale=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return x.to(torch.bfloat16).to(torch.float32).numpy()


def test_constants_match_pages():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        c = json.load(f)
    assert quant.GROUP == c["activation_group"]["value"]
    assert float(quant.AMAX_EPS) == np.float32(c["amax_clamp_min"]["value"])
    assert c["weight_block"]["value"] == [128, 128]


def test_scalar_brute_force_tiny():
    rng = np.random.default_rng(10)
    x = _bf16_values(rng, (3, 384))
    x[1, 128:256] *= 100.0                     # an outlier-scaled group
    x[2, 5] = 40.0                             # one outlier inside a group
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    q, s = quant.per_token_group_quant(x)
    for r in range(x.shape[0]):
        for g in range(3):
            codes, sc = _brute.quant_group_scalar(x[r, 128 * g:128 * (g + 1)])
            assert s[r, g].tobytes() == np.float32(sc).tobytes()
            assert q[r, 128 * g:128 * (g + 1)].tolist() == codes


def test_invariants_random():
    rng = np.random.default_rng(11)
    x = _bf16_values(rng, (64, 1024), scale=3.0)
    q, s = quant.per_token_group_quant(x)
    g = x.reshape(64, 8, 128)
    amax = np.abs(g).max(axis=2).astype(np.float32)
    # scale is exactly float32(amax) / 448 in float32
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    # amax / s rounds to 448, so every group holds a code of magnitude 0x7E
    mags = (q.reshape(64, 8, 128) & 0x7F).max(axis=2)
    assert np.all(mags == 0x7E)
    assert np.all((q & 0x7F) <= 0x7E)          # never NaN
    # dequant error: half an e4m3 ulp of x/s, plus the float32 quotient rounding
    quot = g / s[:, :, None]
    bound = (e4m3.half_ulp(quot) + np.abs(quot) * 2.0 ** -24) * s[:, :, None]
    err = np.abs(quant.dequant(q, s).reshape(64, 8, 128) - g)
    assert np.all(err <= bound * (1 + 1e-9))


def test_special_groups():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, :128] = -0.0
    x[1, 128] = -1e-30                          # rounds to -0 after scaling
    x[1, 129] = 1.0
    q, s = quant.per_token_group_quant(x)
    assert np.all(q[0] == 0)
    assert s[0, 0] == np.float32(1e-8) / np.float32(448.0)
    assert np.all(q[1, :128] == 0x80)           # negative zero keeps its sign
    assert q[1, 128] == 0x80 and q[1, 129] == 0x7E


def test_every_bf16_value_at_unit_scale():
    # a group whose amax is 448 has s == 1 exactly, so q = enc(x): compare
    # with torch's cast on all bf16 values in [-448, 448]
    b = (np.arange(0, 1 << 16, dtype=np.uint32) << 16).view(np.float32)
    b = b[np.isfinite(b) & (np.abs(b) <= 448.0)]
    pad = (-b.size) % 127
    b = np.concatenate([b, np.zeros(pad, dtype=np.float32)]).reshape(-1, 127)
    x = np.concatenate([np.full((b.shape[0], 1), 448.0, np.float32), b], axis=1)
    q, s = quant.per_token_group_quant(x)
    assert np.all(s == 1.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def test_rejects_ragged_k():
    with pytest.raises(ValueError):
        quant.per_token_group_quant(np.zeros((1, 130), dtype=np.float32))


def test_block_dequant_recovers_generator_weights():
    """The generator draws float32 weights and block-quantises them with
    torch; dec(w) * scale must give the drawn weights back within half an
    e4m3 ulp of w/scale times the scale (checks the scale direction and the
    block indexing n // 128, k // 128)."""
    from synth import block_quantize_e4m3
    g = torch.Generator().manual_seed(5)
    w = torch.randn((256, 384), generator=g) * 0.02
    w[:128, 128:256] *= 50.0                    # blocks with very different scales
    codes, scale = block_quantize_e4m3(w)
    wf = quant.block_dequant(codes.numpy(), scale.numpy())
    s_full = np.kron(scale.numpy().astype(np.float64), np.ones((128, 128)))
    quot = w.numpy().astype(np.float64) / s_full
    bound = (e4m3.half_ulp(quot) + np.abs(quot) * 2.0 ** -23) * s_full
    assert np.all(np.abs(wf - w.numpy()) <= bound)
    # a transposed scale grid would break the bound on the scaled blocks
    bad = quant.block_dequant(codes.numpy(), np.ascontiguousarray(scale.numpy()[::-1]))
    assert not np.all(np.abs(bad - w.numpy()) <= bound)
