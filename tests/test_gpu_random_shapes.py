"""GPU parity on seeded random shapes.

The named cases in the other GPU tests pick one shape per branch of the
path.  These draw more shapes from fixed seeds, so that the branches meet
in combinations nobody picked.  The fused forward, 24 shapes: block sizes
16 to 128, with and without the K slices of either GEMM, the one-launch
front end (T <= 16) and the three-kernel one, the slot-parallel and the
one-thread-per-8-outputs combine, raw softmax weights, top_k up to 8 and
experts from 1 to 128, with normal or biased logits; each compared on
every element with the checks of test_gpu_forward.py (routing ids, layout
and activation codes bit for bit, routing weights within 1e-5, requantised
codes through the tie window, the output within the bar).  The dense
block-FP8 linear (12 shapes, every output), grouped top-k with random
expert maps (8 shapes, the checks of test_gpu_routing.py) and the batched
format with random counts (8 shapes, the checks of test_gpu_batched.py),
the MXFP8 layer (8 shapes, the checks of test_gpu_mx_forward.py) and the
MXFP8 linear (8 shapes, every output) likewise."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import linear as ref_linear
from oracle import moe as ref_moe
from synth import make_activations, make_linear, make_mx_linear, make_mx_weights, make_weights
from tests.gpu_util import assert_out_close, note, np_
from tests.test_gpu_batched import _check as _batched_check
from tests.test_gpu_batched import _inputs as _batched_inputs
from tests.test_gpu_forward import _full_case, _layer
from tests.test_gpu_linear import _mx_check as _mx_linear_check
from tests.test_gpu_mx_forward import _check_front as _mx_check_front
from tests.test_gpu_mx_forward import _compare_mx_requant
from tests.test_gpu_mx_forward import _requant_of_pairs as _mx_requant_of_pairs
from tests.test_gpu_mx_forward import _run as _mx_run
from tests.test_gpu_routing import _routed_case

pytestmark = pytest.mark.gpu


def _shapes(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 4, 8, 12, 16, 32, 64, 96, 128]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 2, 3, 5, 7, 11, 16, 17, 31, 64, 100, 255, 300, 513]))
        H = 128 * int(rng.integers(1, 9))
        I = 128 * int(rng.integers(1, 7))
        renorm = bool(rng.integers(0, 2))
        kind = "bias" if rng.integers(0, 3) == 0 else "normal"
        out.append((i, T, H, I, E, k, renorm, kind))
    return out


@pytest.mark.parametrize("i,T,H,I,E,k,renorm,kind", _shapes())
def test_random_shape(i, T, H, I, E, k, renorm, kind):
    w = _layer(T, H, I, E, k, seed=7000 + 13 * i, kind=kind)
    _full_case(w, renorm, what=f"random #{i} ({kind} logits)")


def _linear_shapes(n=12, seed=7331):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 700)), 128 * int(rng.integers(1, 13)), 128 * int(rng.integers(1, 13)))
            for i in range(n)]


@pytest.mark.parametrize("i,M,N,K", _linear_shapes())
def test_random_linear(i, M, N, K):
    """the dense block-FP8 linear on seeded random shapes, every output"""
    x, w, ws = make_linear(M, N, K, seed_base=9000 + 17 * i)
    note(f"random linear #{i} M={M} N={N} K={K}")
    out = moe.fp8_block_linear(x.cuda(), w.cuda(), ws.cuda())
    torch.cuda.synchronize()
    ref, _ = ref_linear.block_fp8_linear(x.float().numpy(), w.numpy(), ws.numpy())
    assert_out_close(np_(out.float()), ref, f"random linear #{i} {M}x{N}x{K}")


def _routed_shapes(n=8, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([4, 8, 12, 16, 32, 64]))
        G = int(rng.choice([d for d in (1, 2, 4, 8) if E % d == 0]))
        kg = 1 if G == 1 else int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(8, kg * (E // G)) + 1))
        T = int(rng.choice([1, 3, 9, 16, 40, 130, 300]))
        H = 128 * int(rng.integers(1, 5))
        I = 128 * int(rng.integers(1, 4))
        local = None
        if rng.integers(0, 3) > 0:           # two in three cases hold a subset of the experts
            n_loc = int(rng.integers(1, E + 1))
            local = sorted(int(v) for v in rng.choice(E, n_loc, replace=False))
        out.append((i, T, H, I, E, k, G, kg, local))
    return out


@pytest.mark.parametrize("i,T,H,I,E,k,G,kg,local", _routed_shapes())
def test_random_routed(i, T, H, I, E, k, G, kg, local):
    """grouped top-k and the expert map on seeded random shapes"""
    _routed_case(T, H, I, E, k, G, kg, local, seed=5000 + 31 * i, what=f"random routed #{i}")


def _batched_shapes(n=8, seed=99):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 13))
        M = int(rng.integers(1, 201))
        H = 128 * int(rng.integers(1, 5))
        I = 128 * int(rng.integers(1, 4))
        counts = [int(c) for c in rng.integers(0, M + 1, E)]
        out.append((i, E, M, H, I, counts))
    return out


@pytest.mark.parametrize("i,E,M,H,I,counts", _batched_shapes())
def test_random_batched(i, E, M, H, I, counts):
    """the batched (masked) expert format on seeded random shapes and counts"""
    counts = np.asarray(counts, np.int32)
    note(f"random batched #{i} E={E} M={M} H={H} I={I} counts={counts.tolist()}")
    x = _batched_inputs(E, M, H, counts, 6000 + i)
    w = make_weights(H, I, E, 6100 + i)
    wsp = torch.empty(moe.moe_fp8_batched_workspace_bytes(E, M, H, I), dtype=torch.uint8, device="cuda")
    out = moe.moe_fp8_batched_experts(x.cuda(), torch.from_numpy(counts).cuda(),
                                      *[a.cuda() for a in w], workspace=wsp)
    torch.cuda.synchronize()
    _batched_check(x, counts, w, out, wsp, E, M, H, I, f"random batched #{i}")


def _mx_layer_shapes(n=8, seed=1717):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 4, 8, 16, 32]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 5, 17, 64, 130, 300]))
        H = 128 * int(rng.integers(1, 7))
        I = 128 * int(rng.integers(2, 7))        # the MXFP8 layer needs I >= 256
        out.append((i, T, H, I, E, k))
    return out


@pytest.mark.parametrize("i,T,H,I,E,k", _mx_layer_shapes())
def test_random_mx_layer(i, T, H, I, E, k):
    """the MXFP8 layer on seeded random shapes, with test_gpu_mx_forward.py's checks"""
    note(f"random mx layer #{i} T={T} H={H} I={I} E={E} k={k}")
    w13, w13e, w2, w2e = make_mx_weights(H, I, E, 8000 + 7 * i)
    x, logits = make_activations(H, E, T, 8100 + 7 * i)
    out, taps = _mx_run(x.cuda(), logits.cuda(), [a.cuda() for a in (w13, w13e, w2, w2e)],
                        T, H, I, E, k)
    ref, info = ref_moe.moe_forward(x.float().numpy(), logits.numpy(), w13.numpy(), w13e.numpy(),
                                    w2.numpy(), w2e.numpy(), k, True, mx=True)
    rows = _mx_check_front(taps, x.float().numpy(), info["ids"], info["w"], E)
    g, ge = _mx_requant_of_pairs(taps, rows, np.arange(T * k), T * k)
    mm, n = _compare_mx_requant(g, ge, info["aq"], info["as"])
    assert mm * n <= 0.01 * n + 3, f"requant mismatch fraction {mm}"
    assert_out_close(np_(out.float()), ref, f"random mx layer #{i}")


def _mx_linear_shapes(n=8, seed=2929):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 700)), 128 * int(rng.integers(1, 13)), 128 * int(rng.integers(2, 13)))
            for i in range(n)]


@pytest.mark.parametrize("i,M,N,K", _mx_linear_shapes())
def test_random_mx_linear(i, M, N, K):
    """the MXFP8 linear on seeded random shapes (K >= 256), every output"""
    x, w, we = make_mx_linear(M, N, K, seed_base=9500 + 11 * i)
    note(f"random mx linear #{i} M={M} N={N} K={K}")
    _mx_linear_check(x, w, we, f"random mx linear #{i} {M}x{N}x{K}")
