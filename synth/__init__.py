"""Seeded synthetic inputs for the fused FP8 MoE layer and the standalone
activation quantiser.

This module is shared by the tests, the benchmark and the smoke check.  It
only draws random numbers and packs them into the layouts the layer takes; it
holds no part of the layer's arithmetic and imports neither the oracle nor
the HIP library.  The FP8 expert weights stand in for a block-quantized
checkpoint: they are drawn N(0, 0.02) and rounded to e4m3fn codes with one
float32 dequant scale per 128x128 block by torch's own float8 conversion.

Workload shapes (named after the model families they imitate; no model
weights or datasets are used):
  tiny     H=256,  I=512,   E=8,   top_k=2, T=16
  mixtral  H=4096, I=14336, E=8,   top_k=2, T=64 / 512, logits = x @ gate^T
  dsv3     H=7168, I=2048,  E=256, top_k=8, T=64 / 8192, logits N(0,1) + b_e,
           b_e = +-0.5 with a seeded sign per expert (load skew)
  qwen3    H=2048, I=768,   E=128, top_k=8, T=1 / 32 / 4096
All route with softmax top-k and renormalisation.  The standalone quant
workload is bf16 [16384, 7168] N(0,1) where 1% of entries (seeded) are
multiplied by 100 in float32 before the one rounding to bf16.

Seeds: seed_base = 1000 * workload_index; +0 activations, +1 logits / gate /
bias, +2 weights (re-seeded per expert, w13 before w2), +3 outlier mask.
"""

import torch

MOE_WORKLOADS = {
    "tiny": dict(index=0, H=256, I=512, E=8, top_k=2, renormalize=True,
                 T=(16,), logits="normal"),
    "mixtral": dict(index=1, H=4096, I=14336, E=8, top_k=2, renormalize=True,
                    T=(64, 512), logits="gate"),
    "dsv3": dict(index=2, H=7168, I=2048, E=256, top_k=8, renormalize=True,
                 T=(64, 8192), logits="bias"),
    "qwen3": dict(index=3, H=2048, I=768, E=128, top_k=8, renormalize=True,
                  T=(1, 32, 4096), logits="normal"),
}
QUANT_WORKLOAD = dict(index=4, M=16384, K=7168, outlier_frac=0.01, outlier_mul=100.0)
# Dense block-FP8 linear: a DeepSeek-V3-shaped dense down projection
# (out features 7168, in features 18432) at a decode and a prefill batch
LINEAR_WORKLOAD = dict(index=5, N=7168, K=18432, M=(64, 8192))
# The same dense shape with MXFP8 operands: [1, 32] blocks, UE8M0 scales
MX_LINEAR_WORKLOAD = dict(index=6, N=7168, K=18432, M=(64, 8192))
MX_BLOCK = 32
# Batched (masked) expert format: the 32 experts of one rank of an 8-way
# DeepSeek-V3 expert placement, up to 256 dispatched rows each, seeded counts
# uniform in [64, 256]
BATCHED_WORKLOAD = dict(index=7, E=32, M=256, H=7168, I=2048, min_count=64)

WEIGHT_STD = 0.02
BLOCK = 128


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def block_quantize_e4m3(w: torch.Tensor):
    """float32 [N, K] -> (uint8 e4m3fn codes [N, K], float32 scales
    [N/128, K/128]) using torch's float8 cast; scale = block amax / 448."""
    N, K = w.shape
    b = w.reshape(N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    amax = b.abs().amax(dim=(1, 3)).clamp_min(1e-8)
    scale = (amax / 448.0).to(torch.float32)
    q = (b / scale[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(N, K).contiguous(), scale.contiguous()


def mx_quantize_e4m3(w: torch.Tensor):
    """float32 [N, K] -> (uint8 e4m3fn codes [N, K], uint8 UE8M0 exponents
    [N, K/32]): a checkpoint stand-in with one power-of-two scale per row and
    32 consecutive columns, the block amax / 448 rounded up to a power of two
    (torch.frexp), and torch's float8 cast of w / scale."""
    N, K = w.shape
    b = w.reshape(N, K // MX_BLOCK, MX_BLOCK)
    amax = b.abs().amax(dim=2).clamp_min(1e-8)
    m, ex = torch.frexp((amax / 448.0).to(torch.float32))
    ex = ex - (m == 0.5).to(ex.dtype)                  # 2^ex >= amax / 448, the least such
    scale = torch.ldexp(torch.ones_like(amax), ex)
    q = (b / scale[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(N, K).contiguous(), (ex + 127).to(torch.uint8).contiguous()


def make_weights(H, I, E, seed, device="cpu", std=WEIGHT_STD):
    """Expert weights: w13 uint8 [E, 2I, H] (rows [0, I) gate, [I, 2I) up),
    w13_scale float32 [E, 2I/128, H/128], w2 uint8 [E, H, I],
    w2_scale float32 [E, H/128, I/128]."""
    if H % BLOCK or I % BLOCK:
        raise ValueError("H and I must be multiples of 128")
    w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=device)
    w13s = torch.empty((E, 2 * I // BLOCK, H // BLOCK), dtype=torch.float32, device=device)
    w2 = torch.empty((E, H, I), dtype=torch.uint8, device=device)
    w2s = torch.empty((E, H // BLOCK, I // BLOCK), dtype=torch.float32, device=device)
    for e in range(E):
        g = _gen(device, seed * 1_000_003 + e)
        a = torch.randn((2 * I, H), generator=g, device=device, dtype=torch.float32) * std
        w13[e], w13s[e] = block_quantize_e4m3(a)
        del a
        b = torch.randn((H, I), generator=g, device=device, dtype=torch.float32) * std
        w2[e], w2s[e] = block_quantize_e4m3(b)
        del b
    return w13, w13s, w2, w2s


def make_activations(H, E, T, seed_base, logits_kind="normal", device="cpu"):
    """x bf16 [T, H] ~ N(0, 1) and router logits float32 [T, E]."""
    gx = _gen(device, seed_base + 0)
    x = torch.randn((T, H), generator=gx, device=device, dtype=torch.float32).to(torch.bfloat16)
    gl = _gen(device, seed_base + 1)
    if logits_kind == "gate":
        gate = torch.randn((E, H), generator=gl, device=device, dtype=torch.float32)
        logits = (x.to(torch.float64) @ gate.to(torch.float64).T).to(torch.float32)
    elif logits_kind == "bias":
        sign = torch.randint(0, 2, (E,), generator=gl, device=device).to(torch.float32) * 2 - 1
        logits = torch.randn((T, E), generator=gl, device=device, dtype=torch.float32) + 0.5 * sign
    else:
        logits = torch.randn((T, E), generator=gl, device=device, dtype=torch.float32)
    return x.contiguous(), logits.contiguous()


def moe_workload(name, T, device="cpu"):
    """All inputs of one named workload at batch T, as a dict of tensors."""
    c = MOE_WORKLOADS[name]
    base = 1000 * c["index"]
    w13, w13s, w2, w2s = make_weights(c["H"], c["I"], c["E"], base + 2, device)
    x, logits = make_activations(c["H"], c["E"], T, base, c["logits"], device)
    return dict(x=x, logits=logits, w13=w13, w13_scale=w13s, w2=w2, w2_scale=w2s,
                H=c["H"], I=c["I"], E=c["E"], T=T, top_k=c["top_k"],
                renormalize=c["renormalize"])


def quant_input(M=None, K=None, device="cpu", seed_base=None,
                outlier_frac=None, outlier_mul=None):
    """bf16 [M, K] N(0, 1) with a seeded fraction of entries scaled up."""
    q = QUANT_WORKLOAD
    M = q["M"] if M is None else M
    K = q["K"] if K is None else K
    seed_base = 1000 * q["index"] if seed_base is None else seed_base
    frac = q["outlier_frac"] if outlier_frac is None else outlier_frac
    mul = q["outlier_mul"] if outlier_mul is None else outlier_mul
    x = torch.randn((M, K), generator=_gen(device, seed_base), device=device,
                    dtype=torch.float32)
    mask = torch.rand((M, K), generator=_gen(device, seed_base + 3), device=device) < frac
    x = torch.where(mask, x * mul, x)
    return x.to(torch.bfloat16).contiguous()


def make_linear(M, N, K, seed_base, device="cpu", std=WEIGHT_STD):
    """Dense linear inputs: x bf16 [M, K] ~ N(0, 1) (seed_base + 0) and a
    weight [N, K] ~ N(0, std) (seed_base + 2), block-quantised to e4m3fn codes
    [N, K] with float32 scales [N/128, K/128]."""
    if N % BLOCK or K % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    x = torch.randn((M, K), generator=_gen(device, seed_base + 0), device=device,
                    dtype=torch.float32).to(torch.bfloat16).contiguous()
    w = torch.randn((N, K), generator=_gen(device, seed_base + 2), device=device,
                    dtype=torch.float32) * std
    wq, ws = block_quantize_e4m3(w)
    return x, wq, ws


def make_mx_linear(M, N, K, seed_base, device="cpu", std=WEIGHT_STD):
    """MXFP8 dense linear inputs: x bf16 [M, K] ~ N(0, 1) (seed_base + 0) and
    a weight [N, K] ~ N(0, std) (seed_base + 2) as e4m3fn codes [N, K] with
    UE8M0 exponent bytes [N, K/32]."""
    if N % 128 or K % 128:
        raise ValueError("N and K must be multiples of 128")
    x = torch.randn((M, K), generator=_gen(device, seed_base + 0), device=device,
                    dtype=torch.float32).to(torch.bfloat16).contiguous()
    w = torch.randn((N, K), generator=_gen(device, seed_base + 2), device=device,
                    dtype=torch.float32) * std
    wq, we = mx_quantize_e4m3(w)
    return x, wq, we


def make_mx_weights(H, I, E, seed, device="cpu", std=WEIGHT_STD):
    """MXFP8 expert weights: w13 uint8 [E, 2I, H] with UE8M0 exponents
    [E, 2I, H/32], w2 uint8 [E, H, I] with exponents [E, H, I/32]; the same
    N(0, std) draws per expert as make_weights, cast with [1, 32] blocks."""
    if H % BLOCK or I % BLOCK:
        raise ValueError("H and I must be multiples of 128")
    w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=device)
    w13e = torch.empty((E, 2 * I, H // MX_BLOCK), dtype=torch.uint8, device=device)
    w2 = torch.empty((E, H, I), dtype=torch.uint8, device=device)
    w2e = torch.empty((E, H, I // MX_BLOCK), dtype=torch.uint8, device=device)
    for e in range(E):
        g = _gen(device, seed * 1_000_003 + e)
        a = torch.randn((2 * I, H), generator=g, device=device, dtype=torch.float32) * std
        w13[e], w13e[e] = mx_quantize_e4m3(a)
        a = torch.randn((H, I), generator=g, device=device, dtype=torch.float32) * std
        w2[e], w2e[e] = mx_quantize_e4m3(a)
        del a
    return w13, w13e, w2, w2e
