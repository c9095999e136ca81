"""Pins of the e4m3fn codec in oracle/e4m3.py against things other than
itself: torch's float8_e4m3fn conversion (an independent library), an
exhaustive nearest-grid-point search, and the half-ulp error bound."""

import numpy as np
import pytest
import torch

from oracle import e4m3
from tests import _brute


def test_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3.decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ref[~nan], got[~nan])


def test_decode_landmarks():
    d = e4m3.decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0x80, 0xFE], dtype=np.uint8))
    assert d.tolist() == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -0.0, -448.0]
    assert np.signbit(d[6])
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)          # codes 0..126 increase strictly


def _midpoint_probe_values():
    grid = _brute.e4m3_grid_torch()
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)   # exact in fp32
    vals = [mids, grid.astype(np.float32)]
    bits = mids.view(np.uint32).astype(np.int64)
    for d in (-2, -1, 1, 2):
        vals.append((bits + d).astype(np.uint32).view(np.float32))
    v = np.concatenate(vals)
    v = v[np.isfinite(v) & (v >= 0)]
    return np.concatenate([v, -v])


def test_encode_brute_force_midpoints():
    v = _midpoint_probe_values()
    assert np.array_equal(e4m3.encode(v), _brute.nearest_codes(v))


def test_encode_brute_force_random():
    rng = np.random.default_rng(1)
    mag = 2.0 ** rng.uniform(-14, 9.5, size=4000)
    v = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    assert np.array_equal(e4m3.encode(v), _brute.nearest_codes(v))


def test_encode_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(2)
    mag = 2.0 ** rng.uniform(-20, 9.6, size=2_000_000)
    v = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    v = np.concatenate([v, _midpoint_probe_values()])
    ref = torch.from_numpy(np.clip(v, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(v), ref)


def test_encode_all_bf16_values():
    # every finite bf16 value (the first quantiser's inputs when s == 1)
    b = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    v = b.view(np.float32)
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(np.clip(v, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(v), ref)


def test_encode_special_values():
    cases = [
        (0.0, 0x00), (-0.0, 0x80), (448.0, 0x7E), (-448.0, 0xFE),
        (1e6, 0x7E), (-1e6, 0xFE), (np.inf, 0x7E), (-np.inf, 0xFE),
        (464.0, 0x7E), (-1e-30, 0x80), (2.0 ** -10, 0x00),
        (3 * 2.0 ** -10, 0x02), (1.0, 0x38), (1.0625, 0x38),   # tie -> even
        (1.1875, 0x3A),                                        # tie -> even
        (2.0 ** -6 * 15 / 16, 0x08),                           # rounds up into the normals
    ]
    v = np.array([c[0] for c in cases], dtype=np.float32)
    assert e4m3.encode(v).tolist() == [c[1] for c in cases]
    assert e4m3.encode(np.array([np.nan], dtype=np.float32))[0] == 0x7F


def test_roundtrip_half_ulp_bound():
    rng = np.random.default_rng(3)
    v = rng.uniform(-448, 448, size=200_000).astype(np.float32)
    v = np.concatenate([v, (rng.standard_normal(100_000) * 1e-2).astype(np.float32)])
    err = np.abs(e4m3.decode(e4m3.encode(v)) - v.astype(np.float64))
    assert np.all(err <= e4m3.half_ulp(v) * (1 + 1e-12))


@pytest.mark.parametrize("mutant", ["ties_away", "no_saturation_clamp"])
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    """A plausible slip in the encoder must fail the pins above."""
    real = e4m3.encode

    def ties_away(v):
        v = np.asarray(v, dtype=np.float32)
        c = real(v)
        # round half away from zero: bump codes that sit on a tie going down
        d = e4m3.decode(c)
        nxt = e4m3.decode(np.minimum((c & 0x7F) + 1, 0x7E).astype(np.uint8))
        tie = np.abs(np.abs(v) - (np.abs(d) + nxt) / 2) == 0
        return np.where(tie & ((c & 0x7F) < 0x7E), c + 1, c).astype(np.uint8)

    def no_clamp(v):
        v = np.asarray(v, dtype=np.float32)
        c = real(v)
        return np.where(np.abs(v) > 464, 0x7F | (c & 0x80), c).astype(np.uint8)

    monkeypatch.setattr(e4m3, "encode", ties_away if mutant == "ties_away" else no_clamp)
    with pytest.raises(AssertionError):
        test_encode_brute_force_midpoints()
        test_encode_special_values()
