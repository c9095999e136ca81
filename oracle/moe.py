"""The fused FP8 block-quantized MoE layer forward, computed literally.

Test infrastructure (see the package docstring).

Sources (vLLM quantization / MoE pages):
  * overview page, "FusedMoE Class": expert weights w13 (gate+up) and w2
    (down) stored [num_experts, N, K]; a top-K router.
  * overview page, "Modular Kernel Architecture": inputs are quantized and
    dispatched, the expert GEMMs run as permute -> GEMM -> unpermute, and the
    results are gathered.
  * overview page, "Triton Fused MoE Kernel": per-block sorted tokens of one
    expert; float32 dequantisation of the quantized accumulation, then the
    optional router-weight multiply.
  * overview page, "Weight Scale Granularities" and the fp8 oracle page's
    quant keys: static 128x128 block weight scales, dynamic per-token
    128-group activation scales, symmetric.
The layer definition adds the activation (SiLU of the gate half times the up
half), the requantisation of that product, and the weighted combine.

Definition, with T tokens, hidden H, intermediate I, E experts, k slots,
pair p = t * k + j routed to expert e = ids[t, j]:
  1. (ids, w) = router.topk_softmax(logits, k, renormalize)
  2. (xq, xs) = quant.per_token_group_quant(x);  Xf = dec(xq) * xs   (float64)
  3. W13f[e] = dec(w13[e]) * w13_scale[e] (block-broadcast, float64), same for W2f
  4. h[p, :] = W13f[e] @ Xf[t]              (float64 matmul), n in [0, 2I)
  5. a[p, i] = silu(h[p, i]) * h[p, I + i]  (rows [0, I) of w13 are the gate,
                                             [I, 2I) the up projection),
     silu(z) = z / (1 + exp(-z)); computed in float64 and rounded to float32,
     the precision in which the requantisation decides its codes
  6. (aq, as) = quant.per_token_group_quant(a)   (group 128 along I)
  7. y[p, :] = W2f[e] @ (dec(aq[p]) * as[p])     (float64 matmul)
  8. out[t, :] = bf16_RNE( sum over j in slot order of w[t, j] * y[t*k+j, :] )
                 summed in float64.
Scale application per 128-wide K block followed by a float32 accumulation
(the way the kernels order it) is the same sum as steps 4 and 7 up to
rounding order.

Parity: routing ids, the sorted layout and the codes/scales of step 2 are
exact targets.  Step 6 codes depend on the accumulation order of steps 4-5,
so they are a diagnostic, not an exact target.  The whole-layer output is
pinned by the special cases in tests/test_oracle_moe.py (E = 1, k = 1 equals
an independently written dense gated MLP; a scalar-loop brute force on a
tiny layer; token-permutation equivariance; the renormalisation identity; a
loose agreement with the unquantized float64 MLP).  The pages print no
numeric example of the layer, so no end-to-end value is pinned to them.
"""

import numpy as np

from . import e4m3, quant, router


def bf16_round(v) -> np.ndarray:
    """float64 -> nearest bfloat16 (ties to even), returned as float32.
    Valid for the normal bf16 range, which is all the layer produces."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                        # v = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # keep 8 significant bits
    return r.astype(np.float32)


def bf16_bits(v32) -> np.ndarray:
    """float32 array holding bf16 values -> uint16 bf16 bit patterns."""
    return (np.ascontiguousarray(v32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(x_rows, w13_e, w13s_e, w2_e, w2s_e):
    """Steps 2-7 for rows that all go to one expert.
    x_rows float32 [n, H] (bf16 values).  Returns dict of per-row tensors."""
    x_rows = np.asarray(x_rows, dtype=np.float32)
    I = w2_e.shape[1]
    xq, xs = quant.per_token_group_quant(x_rows)
    Xf = quant.dequant(xq, xs)
    W13f = quant.block_dequant(w13_e, w13s_e)
    h = Xf @ W13f.T                                       # [n, 2I] float64
    a = (silu(h[:, :I]) * h[:, I:]).astype(np.float32)    # [n, I]
    aq, as_ = quant.per_token_group_quant(a)
    Af = quant.dequant(aq, as_)
    W2f = quant.block_dequant(w2_e, w2s_e)
    y = Af @ W2f.T                                        # [n, H] float64
    return {"xq": xq, "xs": xs, "h": h, "a": a, "aq": aq, "as": as_, "y": y}


def expert_ffn_mx(x_rows, w13_e, w13x_e, w2_e, w2x_e):
    """Steps 2-7 with MXFP8 operands (fp8 oracle API page: block shape
    [1, 32], uint8 UE8M0 scales, activations through the MXFP8 activation
    quant): x and the requantised activation are quantised per row and 32
    columns with power-of-two scales (quant.per_token_group_quant_pow2), the
    weights carry one UE8M0 exponent per row and 32 K elements (w13x_e
    [2I, H/32], w2x_e [H, I/32]).  Otherwise as expert_ffn."""
    x_rows = np.asarray(x_rows, dtype=np.float32)
    I = w2_e.shape[1]
    xq, _, xe = quant.per_token_group_quant_pow2(x_rows, quant.MX_GROUP)
    h = quant.mx_dequant(xq, xe) @ quant.mx_dequant(w13_e, w13x_e).T
    a = (silu(h[:, :I]) * h[:, I:]).astype(np.float32)
    aq, _, ae = quant.per_token_group_quant_pow2(a, quant.MX_GROUP)
    y = quant.mx_dequant(aq, ae) @ quant.mx_dequant(w2_e, w2x_e).T
    return {"xq": xq, "xs": xe, "h": h, "a": a, "aq": aq, "as": ae, "y": y}


def moe_forward(x, logits, w13, w13_scale, w2, w2_scale, top_k: int,
                renormalize: bool, tokens=None, num_expert_group=1, topk_group=1,
                expert_map=None, mx=False):
    """Whole-layer forward.

    x float32 [T, H] (bf16 values), logits float32 [T, E],
    w13 uint8 [E_w, 2I, H], w13_scale float32 [E_w, 2I/128, H/128],
    w2 uint8 [E_w, H, I], w2_scale float32 [E_w, H/128, I/128].
    ``tokens`` optionally restricts the computation to a list of token rows
    (each token's output depends only on its own row, so this gives the same
    values as the full forward at those rows).

    Routing variants: num_expert_group > 1 routes with
    router.grouped_topk_softmax.  ``expert_map`` (int [E], overview page,
    "Expert Parallelism and Expert Maps": global -> local expert index, -1
    for experts held elsewhere) makes the weights those of the E_w local
    experts: a pair routed to expert e runs local expert expert_map[e], and a
    pair whose expert maps to -1 contributes zero ("Triton Fused MoE Kernel":
    zeros are written for such blocks).  The routing weights are those of the
    global routing either way.

    mx=True: the MXFP8 layer (expert_ffn_mx); w13_scale and w2_scale are then
    the weights' UE8M0 exponent bytes [E, 2I, H/32] and [E, H, I/32], and
    info's xs / as hold exponent bytes.

    Returns (out float32 [n_tok, H] holding bf16 values, info dict with ids,
    w, xq, xs and per-pair a, aq, as, y in pair order p = row * k + j)."""
    x = np.asarray(x, dtype=np.float32)
    logits = np.asarray(logits, dtype=np.float32)
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        x = x[tokens]
        logits = logits[tokens]
    T, H = x.shape
    E = logits.shape[1]
    I = w2.shape[2]
    if num_expert_group > 1:
        ids, w = router.grouped_topk_softmax(logits, top_k, num_expert_group, topk_group,
                                             renormalize)
    else:
        ids, w = router.topk_softmax(logits, top_k, renormalize)
    if mx:
        xq, _, xs = quant.per_token_group_quant_pow2(x, quant.MX_GROUP)
    else:
        xq, xs = quant.per_token_group_quant(x)
    ffn = expert_ffn_mx if mx else expert_ffn

    P = T * top_k
    flat = ids.reshape(-1)
    if expert_map is not None:
        expert_map = np.asarray(expert_map, dtype=np.int64)
        flat = expert_map[flat]                  # local expert, -1 where absent
        E = w13.shape[0]
    y = np.zeros((P, H), dtype=np.float64)
    h = np.zeros((P, 2 * I), dtype=np.float64)
    a = np.zeros((P, I), dtype=np.float32)
    aq = np.zeros((P, I), dtype=np.uint8)
    as_ = (np.zeros((P, I // 32), dtype=np.uint8) if mx
           else np.zeros((P, I // 128), dtype=np.float32))
    for e in range(E):
        pairs = np.nonzero(flat == e)[0]
        if pairs.size == 0:
            continue
        r = ffn(x[pairs // top_k], w13[e], w13_scale[e], w2[e], w2_scale[e])
        y[pairs] = r["y"]
        h[pairs] = r["h"]
        a[pairs] = r["a"]
        aq[pairs] = r["aq"]
        as_[pairs] = r["as"]

    acc = np.zeros((T, H), dtype=np.float64)
    for j in range(top_k):
        acc += w[:, j:j + 1].astype(np.float64) * y[j::top_k]
    out = bf16_round(acc)
    info = {"ids": ids, "w": w, "xq": xq, "xs": xs, "h": h, "a": a, "aq": aq,
            "as": as_, "y": y}
    return out, info


def finish_from_requant(aq, as_, ids, w, w2, w2_scale, top_k: int, expert_map=None):
    """Steps 7 and 8 of the definition applied to given requantised
    activations: the second GEMM and the weighted combine, in float64.

    aq uint8 [P, I] and as_ float32 [P, I/128] are the requantised activation
    of every pair p = t * top_k + j (pair order), ids / w the routing [T, k].
    With the oracle's own (aq, as) this is the tail of moe_forward, value for
    value.  It exists because the requantisation of step 6 is a step function
    of a: where a / s lies on a rounding midpoint to within the first GEMM's
    accumulation error, either neighbouring code is a correct result of the
    method (its sums are defined up to rounding order), and the layer's output
    is then this function of the codes actually chosen.

    Returns out float32 [T, H] holding bf16 values."""
    ids = np.asarray(ids)
    T = ids.shape[0]
    H = w2.shape[1]
    flat = ids.reshape(-1)
    if expert_map is not None:
        flat = np.asarray(expert_map, dtype=np.int64)[flat]
    y = np.zeros((T * top_k, H), dtype=np.float64)
    for e in range(w2.shape[0]):
        pairs = np.nonzero(flat == e)[0]
        if pairs.size == 0:
            continue
        Af = quant.dequant(aq[pairs], as_[pairs])
        y[pairs] = Af @ quant.block_dequant(w2[e], w2_scale[e]).T
    acc = np.zeros((T, H), dtype=np.float64)
    for j in range(top_k):
        acc += np.asarray(w)[:, j:j + 1].astype(np.float64) * y[j::top_k]
    return bf16_round(acc)


def batched_experts(x, counts, w13, w13_scale, w2, w2_scale):
    """The expert computation in the batched activation format.

    Source: overview page, "FusedMoEPermuteExpertsUnpermute Implementations"
    (BatchedDeepGemmExperts: the masked grouped GEMM of the FP8 block scheme)
    and the fp8 oracle API page's BatchedExperts activation format; the pages
    define nothing further, so the reading is the plainest one: activations
    already dispatched per expert, x [E, M, H], of which expert e's first
    counts[e] rows are real; each real row goes through that expert's steps
    2-7 (quantise, GEMM1, SiLU*mul, requantise, GEMM2); the routing weights
    belong to the finalize step, not to the experts.

    Returns (out float32 [E, M, H] holding bf16 values, zero at rows
    r >= counts[e], info with the float64 y per expert)."""
    x = np.asarray(x, dtype=np.float32)
    E, M, H = x.shape
    counts = np.asarray(counts, dtype=np.int64)
    out = np.zeros((E, M, H), dtype=np.float32)
    ys = []
    for e in range(E):
        c = int(counts[e])
        if c <= 0:
            ys.append(np.zeros((0, H)))
            continue
        r = expert_ffn(x[e, :c], w13[e], w13_scale[e], w2[e], w2_scale[e])
        out[e, :c] = bf16_round(r["y"])
        ys.append(r["y"])
    return out, {"y": ys}
