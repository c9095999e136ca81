"""The matrix-core rate probe through the C ABI: besides its timing use, its
result has a closed form.  Every MFMA of a wave multiplies the same register
operands, so the sum of all 256 entries of one product is
sum over K of (column sum of A) * (row sum of B), whatever lane holds which
K index (both operands use the same mapping).  The wave's 64 stored floats
then sum to 8 chains x iters x that value."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import e4m3
from tests.gpu_util import note

pytestmark = pytest.mark.gpu


def _expected_wave_sum(kind, iters):
    total = 0.0
    for g in range(4):                        # lane group: lanes 16 g .. 16 g + 15
        lanes = 16 * g + np.arange(16)
        if kind == "f16":
            for i in range(8):                # the lane's eight f16 values
                col_a = np.sum(((lanes + i) & 7) / 128.0)
                row_b = np.sum(((3 * lanes + i) & 7) / 128.0)
                total += col_a * row_b
        else:
            for i in range(8):                # eight dwords = 32 e4m3 values per lane
                for byte in range(4):
                    ca = 0x30 + ((lanes + i) & 7) if byte == 0 else np.full(16, 0x30)
                    cb = 0x28 + ((3 * lanes + i) & 7) if byte == 0 else np.full(16, 0x28)
                    total += (np.sum(e4m3.decode(ca.astype(np.uint8)).astype(np.float64))
                              * np.sum(e4m3.decode(cb.astype(np.uint8)).astype(np.float64)))
    return 8 * iters * total


@pytest.mark.parametrize("kind", ["f16", "fp8"])
def test_probe_closed_form(kind):
    note(f"mfma rate probe {kind}")
    nblocks, iters = 3, 16
    sink = torch.empty(nblocks * 256, dtype=torch.float32, device="cuda")
    flops = moe.moe_mfma_rate_probe(kind, iters, nblocks, sink)
    torch.cuda.synchronize()
    assert flops == nblocks * 4 * iters * 8 * (16384 if kind == "f16" else 65536)
    waves = sink.cpu().numpy().astype(np.float64).reshape(nblocks * 4, 64).sum(axis=1)
    want = _expected_wave_sum(kind, iters)
    # f16 products and sums are exact here (multiples of 2^-14 far below 2^10);
    # the FP8 instruction's own accumulation is held to 1e-6
    rtol = 0.0 if kind == "f16" else 1e-6
    np.testing.assert_allclose(waves, want, rtol=rtol, atol=0)


def test_hbm_read_probe_reads_every_word():
    """The XOR of the probe's per-thread words is the XOR of every 32-bit word
    of the buffer, over a grid that leaves a ragged tail of 16-byte words."""
    note("hbm read probe")
    g = torch.Generator().manual_seed(5)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, ((1 << 20) + 36,), generator=g, dtype=torch.int32)
    nblocks = 7
    sink = torch.zeros(nblocks * 256, dtype=torch.int32, device="cuda")
    n = moe.moe_hbm_read_probe(src.cuda(), nblocks, sink)
    torch.cuda.synchronize()
    assert n == src.numel() * 4
    want = np.bitwise_xor.reduce(src.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
