"""GPU parity of the dense block-FP8 linear (fp8_block_linear through the C
ABI) against oracle/linear.py.

The activation quantiser is the forward's (its codes and scales are exact
targets in tests/test_gpu_stages.py); the product runs on FP8 MFMAs with a
float32 accumulator, whose rounding reaches the bf16 output smoothly, so the
output bar is the layer's: |gpu - ref| <= 1e-2 + 2e-2 |ref| everywhere and a
relative norm error below 1e-2.  The small cases cover every block size the
library picks (16 to 128 rows), a ragged last block, an output width that is
not a multiple of 256 (the stores past it go to the workspace's dump), two K
blocks and a single one; a garbage-filled workspace must not change a bit of
the output.  The full-size DeepSeek-V3-shaped projection is compared on
sampled rows (each output row depends only on its own input row)."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import linear as ref_linear
from synth import LINEAR_WORKLOAD, make_linear
from tests.gpu_util import assert_out_close, note, np_

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [
    (1, 128, 128),      # one row: 16-row blocks
    (5, 256, 384),      # ragged 16-row block
    (20, 384, 256),     # 32-row blocks
    (40, 512, 256),     # 64-row blocks
    (100, 1024, 512),   # 128-row blocks, four K blocks
    (300, 640, 256),    # 128-row blocks, N not a multiple of 256, two K blocks
    (130, 256, 128),    # 128-row blocks with a single K block
])
def test_linear_small(M, N, K):
    x, w, ws = make_linear(M, N, K, seed_base=M + N + K)
    note(f"linear M={M} N={N} K={K}")
    out = moe.fp8_block_linear(x.cuda(), w.cuda(), ws.cuda())
    torch.cuda.synchronize()
    ref, _ = ref_linear.block_fp8_linear(x.float().numpy(), w.numpy(), ws.numpy())
    m = assert_out_close(np_(out.float()), ref, f"linear {M}x{N}x{K}")
    note(f"  max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e}")


def test_linear_workspace_contents_do_not_matter():
    M, N, K = 300, 640, 256
    x, w, ws = make_linear(M, N, K, seed_base=77)
    xd, wd, wsd = x.cuda(), w.cuda(), ws.cuda()
    n = moe.fp8_block_linear_workspace_bytes(M, N, K)
    clean = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dirty = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")   # e4m3 NaN codes everywhere
    note("linear workspace garbage")
    a = moe.fp8_block_linear(xd, wd, wsd, workspace=clean)
    b = moe.fp8_block_linear(xd, wd, wsd, workspace=dirty)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.isfinite(a.float()).all()


@pytest.mark.parametrize("M", LINEAR_WORKLOAD["M"])
def test_linear_full_size(M):
    N, K = LINEAR_WORKLOAD["N"], LINEAR_WORKLOAD["K"]
    x, w, ws = make_linear(M, N, K, 1000 * LINEAR_WORKLOAD["index"], device="cuda")
    note(f"linear full-size M={M} N={N} K={K}")
    out = moe.fp8_block_linear(x, w, ws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).choice(M, min(M, 6), replace=False)]))
    ref, _ = ref_linear.block_fp8_linear(np_(x[torch.from_numpy(rows).cuda()].float()), np_(w), np_(ws))
    m = assert_out_close(np_(out.float())[rows], ref, f"linear full-size M={M}")
    note(f"  sampled {rows.size} rows: max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e}")
