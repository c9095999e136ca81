"""GPU parity of the fused forward on seeded random shapes.

The named cases in test_gpu_forward.py pick one shape per branch of the
path.  These draw 24 more shapes from a fixed seed, so that the branches
meet in combinations nobody picked: block sizes 16 to 128, with and without
the K slices of either GEMM, the one-launch front end (T <= 16) and the
three-kernel one, the slot-parallel and the one-thread-per-8-outputs
combine, raw softmax weights, top_k up to 8 and experts from 1 to 128, with
normal or biased logits.  Each case is compared on every element, with the
checks of test_gpu_forward.py: routing ids, layout and activation codes bit
for bit, routing weights within 1e-5, requantised codes through the tie
window, and the output within the bar."""

import numpy as np
import pytest

from tests.test_gpu_forward import _full_case, _layer

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
