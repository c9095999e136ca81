"""OCP FP8 E4M3 ("e4m3fn") codec, written out from the format's definition.

Test infrastructure (see the package docstring).

The pages fix the FP8 type as e4m3 (``torch.float8_e4m3fn`` /
FLOAT8_E4M3_MAX in the NVFP4 weight-quant code of the "online.nvfp4" API
page); the layer definition fixes round-to-nearest-even with saturation.
The format (OCP 8-bit floating point, E4M3 variant):

  byte c = s eeee mmm, bias 7, no infinities.
  e == 15 and m == 7           -> NaN (0x7F / 0xFF)
  e == 0                       -> (-1)^s * m * 2^-9          (subnormal, incl. +-0)
  otherwise                    -> (-1)^s * (1 + m/8) * 2^(e-7)
  largest finite magnitude     -> 448 = 1.75 * 2^8 (code 0x7E)

``encode`` takes float32 values and returns codes:
  * the sign is kept, so -0.0 and negative values that round to zero give 0x80;
  * magnitudes are clamped to 448 first (saturation);
  * the clamped magnitude is rounded to the nearest point of the E4M3 grid,
    ties going to the even mantissa (an even code).
It works on the float32 bit pattern with integer arithmetic only, so no
intermediate rounding can creep in.  NaN inputs map to 0x7F | sign.

Pinned by tests/test_oracle_e4m3.py: all 256 decodes against the closed form
and against torch's float8_e4m3fn conversion; encode against a brute-force
nearest-grid-point search on every midpoint (and 1-2 float32 ulps either side)
and on random values, against torch's cast after clamping, and the
half-ulp error bound.
"""

import numpy as np

E4M3_MAX = 448.0          # 1.75 * 2**8, the largest finite e4m3fn magnitude
_F32_448_BITS = 0x43E00000  # float32 bit pattern of 448.0


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if (c >> 7) else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 15 and m == 7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * m * 2.0 ** -9
        else:
            out[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_DEC = decode_table()


def decode(codes) -> np.ndarray:
    """codes (uint8 array) -> float64 values."""
    return _DEC[np.asarray(codes, dtype=np.uint8)]


def encode(v) -> np.ndarray:
    """float32 array -> uint8 e4m3fn codes, RNE with saturation at +-448."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    bits = v.view(np.uint32).astype(np.int64)
    sign = (bits >> 31) << 7
    mag = bits & 0x7FFFFFFF
    is_nan = mag > 0x7F800000
    # saturation: any magnitude above 448 (including +inf) becomes 448
    mag = np.minimum(mag, _F32_448_BITS)

    f32_exp = mag >> 23                 # biased float32 exponent
    f32_man = mag & 0x7FFFFF
    code = np.zeros(mag.shape, dtype=np.int64)

    # normal e4m3 range: |v| >= 2^-6, float32 biased exponent >= 127 - 6
    normal = f32_exp >= 121
    e = f32_exp[normal] - 127 + 7       # e4m3 biased exponent, 1..15
    q = f32_man[normal] >> 20           # top 3 mantissa bits
    rem = f32_man[normal] & 0xFFFFF     # the 20 dropped bits
    up = (rem > 0x80000) | ((rem == 0x80000) & ((q & 1) == 1))
    # a mantissa carry out of q = 7 bumps the exponent field by itself
    code[normal] = (e << 3) + q + up.astype(np.int64)

    # subnormal e4m3 range: |v| < 2^-6, value = n * 2^-9 for n in 0..8
    sub = ~normal
    # |v| * 2^9 as an exact binary fraction: significand * 2^(exp-150+9)
    sig = np.where(f32_exp[sub] == 0, f32_man[sub], f32_man[sub] | 0x800000)
    shift = 150 - 9 - np.maximum(f32_exp[sub], 1)   # >= 150-9-120 = 21
    shift = np.minimum(shift, 62)
    n = sig >> shift
    frac = sig - (n << shift)
    half = np.int64(1) << (shift - 1)
    up = (frac > half) | ((frac == half) & ((n & 1) == 1))
    code[sub] = n + up.astype(np.int64)     # n = 8 is code 0x08 = 2^-6, correct

    code = np.where(is_nan, 0x7F, code)
    return (code | sign).astype(np.uint8)


def half_ulp(v) -> np.ndarray:
    """Half the spacing of the e4m3 grid at |v| (float64), for |v| <= 448."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)
