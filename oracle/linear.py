"""The dense block-FP8 linear layer, computed literally.

Test infrastructure (see the package docstring).

Source: overview page, "W8A8BlockFp8LinearOp - Block FP8 GEMM Dispatch"
(the block-wise FP8 GEMM of DeepSeek-V3-style dense layers) with the scale
granularities of "Weight Scale Granularities" (a dynamic scale per 128
elements of each activation row, a static scale per 128x128 weight block).

Definition, for x [M, K] (bf16 values), codes w [N, K], scales
w_scale [N/128, K/128]:
  1. (xq, xs) = quant.per_token_group_quant(x);  Xf = dec(xq) * xs (float64)
  2. Wf = dec(w) * w_scale, broadcast over each 128x128 block (float64)
  3. out = bf16_RNE(Xf @ Wf^T)
Applying the two scales per 128-wide K block to each block's partial sum
(the kernels' order) is the same sum up to rounding order.

The MXFP8 linear (mxfp8_linear): fp8 oracle API page, the MXFP8 block shape
[1, 32] with uint8 UE8M0 activation scales [num_tokens, hidden / 32], and
the overview page's "DeepGEMM Scale Formats" (power-of-two scales as UE8M0
exponent bytes).  Both operands carry one power-of-two scale per row and 32
consecutive K elements:
  1. (xq, xs, xe) = quant.per_token_group_quant_pow2(x, 32)
     Xf[m, k] = dec(xq[m, k]) * 2^(xe[m, k/32] - 127)   (float64)
  2. Wf[n, k] = dec(w[n, k]) * 2^(w_e[n, k/32] - 127)   (float64)
  3. out = bf16_RNE(Xf @ Wf^T)

Parity: pinned in tests/test_oracle_linear.py by a brute force with explicit
per-K-block scale indexing, a closed form (unit scales and e4m3-exact
activations give an exact integer product), row-permutation equivariance,
the effect of scaling the weight scales, and a loose match to the
unquantised float64 product; the MXFP8 form by a scalar brute force over
32-wide blocks with planted mistakes (a 128-wide scale block, transposed
exponent indexing), exponent covariance and the unquantised product.
"""

import numpy as np

from . import quant
from .moe import bf16_round


def block_fp8_linear(x, w, w_scale):
    """x float32 [M, K] holding bf16 values, w uint8 [N, K], w_scale float32
    [N/128, K/128].  Returns (out float32 [M, N] holding bf16 values, info
    with xq, xs and the float64 product before rounding)."""
    x = np.asarray(x, dtype=np.float32)
    xq, xs = quant.per_token_group_quant(x)
    Xf = quant.dequant(xq, xs)
    Wf = quant.block_dequant(w, w_scale)
    acc = Xf @ Wf.T
    return bf16_round(acc), {"xq": xq, "xs": xs, "acc": acc}


mx_dequant = quant.mx_dequant


def mxfp8_linear(x, w, w_e):
    """x float32 [M, K] holding bf16 values, w uint8 [N, K], w_e uint8
    [N, K/32].  Returns (out float32 [M, N] holding bf16 values, info with xq,
    xe and the float64 product before rounding)."""
    x = np.asarray(x, dtype=np.float32)
    xq, _, xe = quant.per_token_group_quant_pow2(x, quant.MX_GROUP)
    acc = mx_dequant(xq, xe) @ mx_dequant(w, w_e).T
    return bf16_round(acc), {"xq": xq, "xe": xe, "acc": acc}
