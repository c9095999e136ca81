"""Pins of the power-of-two-scale quantiser (oracle/quant.py,
per_token_group_quant_pow2 and ceil_pow2).

* ceil_pow2 against its definition: exact powers of two map to themselves,
  any other float32 to the next power of two (checked on its bits, and on
  the neighbours of powers of two);
* a scalar brute force: the float32 scale of each group rounded up with
  Python's exact log2 of powers of two, codes by exhaustive nearest search
  over torch's e4m3 grid;
* invariants: no code saturates, every group holds a code of at least half the
  range (the scale is less than twice the float32 scale), the UE8M0 byte
  decodes to the scale, and an all-zero row gets the scale of the 1e-8 floor;
* where max(amax, 1e-8) / 448 is itself a power of two the codes equal those
  of the float32-scale quantiser;
* a planted mistake (rounding the scale down) fails the brute force.
"""

import math

import numpy as np
import pytest
import torch

from oracle import e4m3, quant
from synth import quant_input
from tests import _brute


def test_ceil_pow2_definition():
    k = np.arange(-40, 21)
    p = np.ldexp(np.float32(1), k).astype(np.float32)
    assert np.array_equal(quant.ceil_pow2(p), p)
    above = np.nextafter(p, np.float32(np.inf))
    assert np.array_equal(quant.ceil_pow2(above), (p * 2).astype(np.float32))
    rng = np.random.default_rng(2)
    s = np.exp(rng.uniform(np.log(1e-12), np.log(1e6), 100_000)).astype(np.float32)
    r = quant.ceil_pow2(s)
    bits = r.view(np.uint32)
    assert np.all(bits & 0x7FFFFF == 0)
    assert np.all(r >= s) and np.all(r.astype(np.float64) / 2 < s)


def _brute_group(vals, round_down=False):
    amax = np.float32(0)
    for v in vals:
        if abs(np.float32(v)) > amax:
            amax = np.float32(abs(np.float32(v)))
    s32 = np.float32(max(amax, np.float32(1e-8))) / np.float32(448)
    lg = math.log2(float(s32))
    p = 2.0 ** (math.floor(lg) if round_down else math.ceil(lg))
    codes = [_brute.nearest_code(np.float32(np.float32(v) / np.float32(p))) for v in vals]
    return codes, np.float32(p)


@pytest.mark.parametrize("group", [32, 128])
def test_matches_brute_force(group):
    x = quant_input(M=3, K=256, seed_base=31).float().numpy()
    q, s, ex = quant.per_token_group_quant_pow2(x, group)
    for r in range(x.shape[0]):
        for g in range(x.shape[1] // group):
            codes, p = _brute_group(x[r, group * g:group * (g + 1)])
            assert list(q[r, group * g:group * (g + 1)]) == codes
            assert s[r, g] == p


@pytest.mark.parametrize("group", [32, 128])
def test_invariants(group):
    x = quant_input(M=8, K=512, seed_base=41).float().numpy()
    q, s, ex = quant.per_token_group_quant_pow2(x, group)
    d = e4m3.decode(q).reshape(8, -1, group)
    assert np.all(np.abs(d) <= 448) and not np.any((q & 0x7F) == 0x7F)
    assert np.all(np.max(np.abs(d), axis=2) >= 224)   # amax/s in (224, 448]; the grid steps by 16 there
    assert np.array_equal(np.ldexp(1.0, ex.astype(np.int64) - 127).astype(np.float32), s)
    err = np.abs(d * s[:, :, None] - x.reshape(8, -1, group))
    bound = e4m3.half_ulp(x.reshape(8, -1, group) / s[:, :, None]) * s[:, :, None]
    assert np.all(err <= bound)
    zq, zs, _ = quant.per_token_group_quant_pow2(np.zeros((1, group), np.float32), group)
    assert np.all(zq == 0) and zs[0, 0] == np.float32(2.0 ** -35)   # ceil(1e-8 / 448) = 2^-35


def test_equal_to_float32_scales_when_already_a_power_of_two():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(4, 256)).astype(np.float32)
    x[:, ::128] = np.float32(448 * 2.0 ** -3)          # group amax 56: float32 scale 2^-3 exactly
    x = np.clip(x, -55, 55); x[:, ::128] = 56.0
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    q2, s2, _ = quant.per_token_group_quant_pow2(x, 128)
    q1, s1 = quant.per_token_group_quant(x, 128)
    assert np.array_equal(s1, s2) and np.array_equal(q1, q2)


def test_planted_round_down_fails():
    x = quant_input(M=1, K=128, seed_base=51).float().numpy()
    q, s, _ = quant.per_token_group_quant_pow2(x, 128)
    codes, p = _brute_group(x[0], round_down=True)
    assert s[0, 0] != p or list(q[0]) != codes


def test_float32_scales_group_32_brute_force():
    # the float32-scale quantiser at group 32 (the other formats' float32 s)
    x = quant_input(M=2, K=128, seed_base=61).float().numpy()
    q, s = quant.per_token_group_quant(x, 32)
    for r in range(2):
        for g in range(4):
            codes, sc = _brute.quant_group_scalar(x[r, 32 * g:32 * (g + 1)])
            assert list(q[r, 32 * g:32 * (g + 1)]) == codes and s[r, g] == sc


def test_mx_constants_match_pages():
    import json
    import os
    from synth import MX_BLOCK
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")) as f:
        c = json.load(f)
    assert [1, quant.MX_GROUP] == c["mxfp8_block"]["value"] and MX_BLOCK == quant.MX_GROUP
    # row-major exponent bytes read as little-endian int32 words: four groups per word
    e = np.arange(8, dtype=np.uint8).reshape(1, 8) + 120
    words = e.view("<u4")
    assert words.shape == (1, 8 // c["ue8m0_values_per_int32"]["value"])
    assert [(int(words[0, 1]) >> (8 * i)) & 0xFF for i in range(4)] == list(range(124, 128))
