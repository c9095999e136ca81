"""CPU tests of the binding's shape checks: every wrapper compares the full
shape of each tensor with what the C ABI will assume (x [T, H], router logits
[T, E], w13 [E, 2I, H] with scales [E, 2I/128, H/128], w2 [E, H, I] with
scales [E, H/128, I/128], out [T, H], and the like for the other entry
points) and raises ValueError before any pointer reaches the library, so a
mismatched tensor can never make a kernel read or write past its allocation.
The tensors here live on the CPU: a call that passed the shape checks would
stop at the device check (TypeError), so no test here can launch anything."""

import pytest
import torch

import fp8_block_quantized_amd as moe

T, H, I, E, K = 4, 384, 128, 8, 2


def _moe(**over):
    a = dict(x=torch.zeros((T, H), dtype=torch.bfloat16),
             router_logits=torch.zeros((T, E)),
             w13=torch.zeros((E, 2 * I, H), dtype=torch.uint8),
             w13_scale=torch.zeros((E, 2 * I // 128, H // 128)),
             w2=torch.zeros((E, H, I), dtype=torch.uint8),
             w2_scale=torch.zeros((E, H // 128, I // 128)))
    a.update(over)
    return a


def _call_forward(a, **kw):
    return moe.moe_fp8_forward(a["x"], a["router_logits"], a["w13"], a["w13_scale"], a["w2"],
                               a["w2_scale"], K, True, **kw)


def test_forward_well_shaped_reaches_the_device_check():
    with pytest.raises(TypeError):
        _call_forward(_moe())


@pytest.mark.parametrize("name,shape", [
    ("x", (T, H + 128)), ("x", (T + 1, H)), ("x", (T, H, 1)), ("x", (T, 200)),
    ("router_logits", (T + 1, E)), ("router_logits", (T,)),
    ("w13", (E, 2 * I, H + 128)), ("w13", (E, 2 * I + 128, H)), ("w13", (E + 1, 2 * I, H)),
    ("w13_scale", (E, 2 * I // 128, H // 128 + 1)), ("w13_scale", (E, H // 128, 2 * I // 128)),
    ("w2", (E, H, I + 128)), ("w2", (E + 1, H, I)), ("w2", (E, H + 128, I)),
    ("w2_scale", (E, H // 128 + 1, I // 128)), ("w2_scale", (E - 1, H // 128, I // 128)),
])
def test_forward_rejects_each_mismatched_tensor(name, shape):
    dtype = _moe()[name].dtype
    with pytest.raises(ValueError):
        _call_forward(_moe(**{name: torch.zeros(shape, dtype=dtype)}))


def test_forward_rejects_experts_differing_from_the_logits():
    # weights for 4 experts but logits over 8: without an expert map they must agree
    a = _moe(w13=torch.zeros((4, 2 * I, H), dtype=torch.uint8),
             w13_scale=torch.zeros((4, 2 * I // 128, H // 128)),
             w2=torch.zeros((4, H, I), dtype=torch.uint8),
             w2_scale=torch.zeros((4, H // 128, I // 128)))
    with pytest.raises(ValueError):
        _call_forward(a)


def test_forward_rejects_a_wrong_output():
    with pytest.raises(ValueError):
        _call_forward(_moe(), out=torch.zeros((T, H - 128), dtype=torch.bfloat16))


def test_routed_checks_local_weights_and_map():
    a = _moe()
    # local weights: w2 must hold as many experts as w13
    bad = dict(a, w2=torch.zeros((3, H, I), dtype=torch.uint8))
    with pytest.raises(ValueError):
        moe.moe_fp8_forward_routed(bad["x"], bad["router_logits"], bad["w13"], bad["w13_scale"],
                                   bad["w2"], bad["w2_scale"], K, True,
                                   expert_map=torch.zeros(E, dtype=torch.int32))
    with pytest.raises(ValueError):     # the map covers the E global experts
        moe.moe_fp8_forward_routed(a["x"], a["router_logits"], a["w13"], a["w13_scale"], a["w2"],
                                   a["w2_scale"], K, True,
                                   expert_map=torch.zeros(E - 1, dtype=torch.int32))
    with pytest.raises(TypeError):      # well shaped: stops at the device check
        moe.moe_fp8_forward_routed(a["x"], a["router_logits"], a["w13"], a["w13_scale"], a["w2"],
                                   a["w2_scale"], K, True,
                                   expert_map=torch.zeros(E, dtype=torch.int32))


def test_mx_forward_checks_exponent_shapes():
    Im = 256                             # the MXFP8 layer needs two K blocks in GEMM2
    a = _moe(w13=torch.zeros((E, 2 * Im, H), dtype=torch.uint8),
             w13_scale=torch.zeros((E, 2 * Im, H // 32), dtype=torch.uint8),
             w2=torch.zeros((E, H, Im), dtype=torch.uint8),
             w2_scale=torch.zeros((E, H, Im // 32), dtype=torch.uint8))
    call = lambda b: moe.moe_fp8_mx_forward(b["x"], b["router_logits"], b["w13"], b["w13_scale"],
                                            b["w2"], b["w2_scale"], K, True)
    with pytest.raises(TypeError):
        call(a)
    with pytest.raises(ValueError):
        call(dict(a, w13_scale=torch.zeros((E, 2 * Im // 128, H // 128))))
    with pytest.raises(ValueError):
        call(dict(a, w2_scale=torch.zeros((E, H, Im // 32 + 1), dtype=torch.uint8)))


def test_batched_checks():
    M = 16
    x = torch.zeros((E, M, H), dtype=torch.bfloat16)
    cnt = torch.zeros(E, dtype=torch.int32)
    w = [torch.zeros((E, 2 * I, H), dtype=torch.uint8), torch.zeros((E, 2 * I // 128, H // 128)),
         torch.zeros((E, H, I), dtype=torch.uint8), torch.zeros((E, H // 128, I // 128))]
    with pytest.raises(TypeError):
        moe.moe_fp8_batched_experts(x, cnt, *w)
    with pytest.raises(ValueError):
        moe.moe_fp8_batched_experts(x, torch.zeros(E + 1, dtype=torch.int32), *w)
    with pytest.raises(ValueError):
        moe.moe_fp8_batched_experts(x, cnt, w[0], w[1], torch.zeros((E, H, 2 * I), dtype=torch.uint8),
                                    w[3])
    with pytest.raises(ValueError):
        moe.moe_fp8_batched_experts(x, cnt, *w, out=torch.zeros((E, M + 1, H), dtype=torch.bfloat16))


@pytest.mark.parametrize("fn,scale", [
    (moe.fp8_block_linear, lambda N, K: torch.zeros((N // 128, K // 128))),
    (moe.mxfp8_linear, lambda N, K: torch.zeros((N, K // 32), dtype=torch.uint8)),
])
def test_linear_checks(fn, scale):
    M, N, Kd = 8, 256, 512
    x = torch.zeros((M, Kd), dtype=torch.bfloat16)
    w = torch.zeros((N, Kd), dtype=torch.uint8)
    with pytest.raises(TypeError):
        fn(x, w, scale(N, Kd))
    with pytest.raises(ValueError):
        fn(x, torch.zeros((N, Kd + 128), dtype=torch.uint8), scale(N, Kd + 128))
    with pytest.raises(ValueError):
        fn(x, w, scale(N + 128, Kd))
    with pytest.raises(ValueError):
        fn(x, w, scale(N, Kd), out=torch.zeros((M, N + 128), dtype=torch.bfloat16))


def test_quant_and_router_checks():
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.per_token_group_quant_fp8(x, q=torch.zeros((4, 128), dtype=torch.uint8))
    with pytest.raises(ValueError):
        moe.per_token_group_quant_fp8(x, scales=torch.zeros((4, 1)))
    with pytest.raises(ValueError):
        moe.per_token_group_quant_fp8(torch.zeros((4, 200), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        moe.per_token_group_quant_fp8_fmt(x, 32, "ue8m0", scales=torch.zeros((4, 4), dtype=torch.uint8))
    with pytest.raises(ValueError):
        moe.per_token_group_quant_fp8_fmt(x, 64)
    lg = torch.zeros((4, 8))
    with pytest.raises(ValueError):
        moe.moe_topk_softmax(lg, 2, True, ids=torch.zeros((4, 3), dtype=torch.int32))
    with pytest.raises(ValueError):
        moe.moe_topk_softmax_grouped(lg, 2, 2, 1, True, weights=torch.zeros((5, 2)))
