"""Brute-force helpers for the oracle pins.  They share nothing with the
oracle: the e4m3 grid comes from torch's float8_e4m3fn conversion, and the
nearest point is found by exhaustive search over all finite codes."""

import numpy as np
import torch


def e4m3_grid_torch() -> np.ndarray:
    """float64 value of codes 0..126 (the finite non-negative magnitudes),
    as torch converts them."""
    codes = torch.arange(0, 127, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


_GRID = e4m3_grid_torch()


def nearest_code(v) -> int:
    """Scalar float32 value -> code by exhaustive nearest search over the
    grid (ties to the even code), saturating at 448, sign kept."""
    v = np.float32(v)
    neg = bool(np.signbit(v))
    a = min(abs(float(v)), 448.0)
    d = np.abs(_GRID - a)
    best = d.min()
    cands = [c for c in range(127) if d[c] == best]
    if len(cands) == 1:
        c = cands[0]
    else:
        assert len(cands) == 2
        c = cands[0] if cands[0] % 2 == 0 else cands[1]
    return c | (0x80 if neg else 0)


def nearest_codes(vals) -> np.ndarray:
    vals = np.asarray(vals, dtype=np.float32).ravel()
    return np.array([nearest_code(v) for v in vals], dtype=np.uint8)


def quant_group_scalar(row) -> tuple:
    """One 128-group quantised with scalar float32 arithmetic and the
    brute-force encoder: (codes list, scale)."""
    xs = [np.float32(v) for v in row]
    amax = np.float32(0.0)
    for v in xs:
        if abs(v) > amax:
            amax = np.float32(abs(v))
    s = np.float32(max(amax, np.float32(1e-8))) / np.float32(448.0)
    codes = [nearest_code(np.float32(v / s)) for v in xs]
    return codes, np.float32(s)
