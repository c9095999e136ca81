"""Per-token, per-group dynamic FP8 activation quantisation (group 128).

Test infrastructure (see the package docstring).

Sources: the fp8 oracle API page fixes the activation quant key as dynamic,
symmetric, 128-element groups per token ("kFp8Dynamic128Sym"), with static
128x128 block weight scales; the "Weight Scale Granularities" section of the
overview page defines GROUP scales as one scale per 128 consecutive
elements.  The layer definition fixes scale = amax / 448 and round-to-
nearest-even.  Scales are dequant multipliers (x ~= dec(q) * s), the
convention the fp8 oracle page uses for its dequant alphas
(w_scale * a_scale) and the NVFP4 page uses for its stored weight scale
(amax / (fp4_max * fp8_max)).  The amax guard is the 1e-8 lower clamp that
the NVFP4 weight quantiser applies to its amax.

Definition, for each row r and group g of 128 consecutive columns:
  xg   = float32(x[r, 128g : 128g+128])
  amax = max |xg|                                   (exact)
  s    = float32(max(amax, 1e-8)) / float32(448)    (IEEE float32, RNE)
  q[i] = e4m3.encode(float32(xg[i]) / s)            (IEEE float32 RNE divide,
                                                     then clamp to +-448 and
                                                     one RNE onto the grid)
The quotient is rounded to float32 before the e4m3 rounding: that double
rounding is part of the definition, and the GPU takes the same float32
decision.

Pinned by tests/test_oracle_quant.py (scalar brute-force loop, invariants
on the maximum code, the exact scale, the dequant error bound and the
all-zero and negative-zero cases).  per_token_group_quant_pow2 (power-of-two
scales, groups of 32 or 128) is pinned in tests/test_oracle_quant_pow2.py.
"""

import numpy as np

from . import e4m3

GROUP = 128
MX_GROUP = 32          # the MXFP8 [1, 32] block: one UE8M0 scale per 32 elements
AMAX_EPS = np.float32(1e-8)
FP8_MAX = np.float32(448.0)


def per_token_group_quant(x, group: int = GROUP):
    """x: [M, K] array of float32-representable values (bf16 inputs are exact
    in float32).  Returns (q uint8 [M, K], s float32 [M, K // group])."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    xg = x.reshape(M, K // group, group)
    amax = np.max(np.abs(xg), axis=2)
    s = np.maximum(amax, AMAX_EPS).astype(np.float32) / FP8_MAX
    s = s.astype(np.float32)
    quot = (xg / s[:, :, None]).astype(np.float32)
    q = e4m3.encode(quot).reshape(M, K)
    return q, s


def dequant(q, s, group: int = GROUP) -> np.ndarray:
    """float64 dequantised values dec(q) * s, broadcast per group."""
    q = np.asarray(q, dtype=np.uint8)
    M, K = q.shape
    d = e4m3.decode(q).reshape(M, K // group, group)
    return (d * np.asarray(s, dtype=np.float64)[:, :, None]).reshape(M, K)


def block_dequant(w, ws, block: int = 128) -> np.ndarray:
    """Static 2-D block weights: w uint8 [N, K] codes, ws float32
    [N/block, K/block] dequant multipliers -> float64 [N, K] with
    W[n, k] = dec(w[n, k]) * ws[n // block, k // block]."""
    w = np.asarray(w, dtype=np.uint8)
    N, K = w.shape
    d = e4m3.decode(w)
    scale = np.repeat(np.repeat(np.asarray(ws, dtype=np.float64), block, axis=0),
                      block, axis=1)
    return d * scale


def ceil_pow2(s) -> np.ndarray:
    """float32 s > 0 -> the smallest power of two >= s, as float32: the scale
    rounded up to an unsigned 8-bit exponent with no mantissa (UE8M0)."""
    s = np.asarray(s, dtype=np.float32)
    m, e = np.frexp(s.astype(np.float64))          # s = m * 2^e, 0.5 <= m < 1
    return np.where(m == 0.5, s.astype(np.float64), np.ldexp(1.0, e)).astype(np.float32)


def per_token_group_quant_pow2(x, group: int = GROUP):
    """Power-of-two group scales.

    Sources: overview page, "DeepGEMM Scale Formats" (FLOAT32_CEIL_UE8M0:
    float32 scales rounded up to UE8M0; UE8M0: the same exponents packed as
    bytes, four per int32); fp8 oracle API page, the MXFP8 [1, 32] block
    shape whose activation scales are uint8 UE8M0 values laid out
    (num_tokens, hidden // 32).  Definition, per row and group of `group`
    (32 or 128) consecutive columns:
      s = ceil_pow2(float32(max(amax, 1e-8)) / 448)    (the float32 scale of
                                                         per_token_group_quant,
                                                         rounded up)
      q = e4m3.encode(float32(x / s))                   (exact: s is a power of two)
      e = log2(s) + 127                                 (the UE8M0 byte)
    Rounding up keeps |x / s| <= 448, so no value saturates.
    Returns (q uint8 [M, K], s float32 [M, K // group], e uint8 [M, K // group])."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    xg = x.reshape(M, K // group, group)
    amax = np.max(np.abs(xg), axis=2)
    s = ceil_pow2((np.maximum(amax, AMAX_EPS).astype(np.float32) / FP8_MAX).astype(np.float32))
    quot = (xg / s[:, :, None]).astype(np.float32)
    q = e4m3.encode(quot).reshape(M, K)
    ex = (np.frexp(s.astype(np.float64))[1] - 1 + 127).astype(np.uint8)
    return q, s, ex


def mx_dequant(q, e, block: int = MX_GROUP) -> np.ndarray:
    """uint8 codes [R, K], UE8M0 exponent bytes [R, K/block] -> float64
    [R, K] with value dec(q[r, k]) * 2^(e[r, k // block] - 127)."""
    q = np.asarray(q, dtype=np.uint8)
    R, K = q.shape
    d = e4m3.decode(q).reshape(R, K // block, block)
    p = np.ldexp(1.0, np.asarray(e, dtype=np.int64) - 127)
    return (d * p[:, :, None]).reshape(R, K)
