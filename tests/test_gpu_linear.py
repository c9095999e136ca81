"""GPU parity of the dense block-FP8 linear (fp8_block_linear through the C
ABI) and the MXFP8 linear (mxfp8_linear) against oracle/linear.py.

The activation quantiser is the forward's (its codes and scales are exact
targets in tests/test_gpu_stages.py); the product runs on FP8 MFMAs with a
float32 accumulator, whose rounding reaches the bf16 output smoothly, so the
output bar is the layer's: |gpu - ref| <= 1e-2 + 2e-2 |ref| everywhere and a
relative norm error below 1e-2.  The small cases cover one and several
128-row blocks, ragged last blocks from 1 to 65 rows (the rows past M are
the workspace's padding rows), an output width that is not a multiple of
256 (the stores past it go to the workspace's dump), K split into slices
(including counts of K blocks that do not divide evenly) and not, two K
blocks and a single one; a garbage-filled workspace must not change a bit
of the output, with many padding rows or few.  A 4096 x 4096 x 1024 case has 512 output tiles
against one persistent workgroup per CU, so each workgroup runs two tiles
back to back (the hand-counted waits between one tile's stores and the next
tile's loads); it is compared on every output.  The MXFP8 cases add
exponents drawn at random per 32-element block on both operands, so that a
scale applied to the wrong block shows as a factor of a power of two.  The
full-size DeepSeek-V3-shaped projection is compared on every output at
M = 64, and on 32 sampled rows at M = 8192 (2.2 TFLOP in the oracle; each
output row depends only on its own input row)."""

import numpy as np
import pytest
import torch

import fp8_block_quantized_amd as moe
from oracle import linear as ref_linear
from synth import LINEAR_WORKLOAD, MX_LINEAR_WORKLOAD, make_linear, make_mx_linear
from tests.gpu_util import assert_out_close, note, np_

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [
    (1, 128, 128),      # one row, one K block
    (5, 256, 384),      # ragged block, three K blocks
    (20, 384, 256),
    (40, 512, 256),
    (16, 256, 1024),    # eight K blocks split into slices
    (33, 128, 2048),
    (64, 384, 1152),    # nine K blocks split into three slices
    (65, 256, 512),
    (100, 1024, 512),   # 128-row blocks, four K blocks
    (300, 640, 256),    # 128-row blocks, N not a multiple of 256, two K blocks
    (130, 256, 128),    # 128-row blocks with a single K block
    (4096, 4096, 1024), # 512 tiles: two per persistent workgroup, eight K blocks
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


def test_linear_small_m_workspace_contents_do_not_matter():
    """A 128-row block that is almost all padding rows (read from the
    workspace, never stored), with K split into slices."""
    M, N, K = 5, 384, 1024
    x, w, ws = make_linear(M, N, K, seed_base=79)
    xd, wd, wsd = x.cuda(), w.cuda(), ws.cuda()
    n = moe.fp8_block_linear_workspace_bytes(M, N, K)
    clean = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dirty = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    note("linear small-M workspace garbage")
    a = moe.fp8_block_linear(xd, wd, wsd, workspace=clean)
    b = moe.fp8_block_linear(xd, wd, wsd, workspace=dirty)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref, _ = ref_linear.block_fp8_linear(x.float().numpy(), w.numpy(), ws.numpy())
    assert_out_close(np_(a.float()), ref, "linear small-M garbage workspace")


def _rows(M, seed):
    """every row at decode sizes; the first, the last and 30 random rows otherwise"""
    if M <= 64:
        return np.arange(M)
    return np.unique(np.concatenate([[0, M - 1], np.random.default_rng(seed).choice(M, 30, replace=False)]))


@pytest.mark.parametrize("M", LINEAR_WORKLOAD["M"])
def test_linear_full_size(M):
    N, K = LINEAR_WORKLOAD["N"], LINEAR_WORKLOAD["K"]
    x, w, ws = make_linear(M, N, K, 1000 * LINEAR_WORKLOAD["index"], device="cuda")
    note(f"linear full-size M={M} N={N} K={K}")
    out = moe.fp8_block_linear(x, w, ws)
    torch.cuda.synchronize()
    rows = _rows(M, M)
    ref, _ = ref_linear.block_fp8_linear(np_(x[torch.from_numpy(rows).cuda()].float()), np_(w), np_(ws))
    m = assert_out_close(np_(out.float())[rows], ref, f"linear full-size M={M}")
    note(f"  {rows.size} rows: max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e}")


# ---- MXFP8 ----

def _mx_spread(M, N, K, seed):
    """x bf16 N(0, 1) with each 32-group scaled by 2^u, u in [-6, 6]; weight
    codes from N(0, 112) cast to e4m3 and exponent bytes 115 + [-4, 4],
    both drawn per 32-element block."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x = x * torch.pow(2.0, torch.randint(-6, 7, (M, K // 32, 1), generator=g).float()).expand(M, K // 32, 32).reshape(M, K)
    w = (torch.randn((N, K), generator=g) * 112.0).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    we = (115 + torch.randint(-4, 5, (N, K // 32), generator=g)).to(torch.uint8)
    return x.to(torch.bfloat16).contiguous(), w.contiguous(), we.contiguous()


# error of the scaled FP8 MFMA's accumulation, relative to the sum of the
# magnitudes of the products it adds (measured up to 1.3e-4 on full-range codes)
MX_MFMA_ERR = 2.0 ** -12


def _mx_check(x, w, we, what, spread=False):
    """The output bar; with spread exponents (operand blocks up to 2^10
    apart, built to expose a misapplied exponent) the scaled MFMA's own
    accumulation error, MX_MFMA_ERR of the sum of |products|, is allowed on
    top of it elementwise, and the relative norm error must still be < 1e-2."""
    out = moe.mxfp8_linear(x.cuda(), w.cuda(), we.cuda())
    torch.cuda.synchronize()
    ref, info = ref_linear.mxfp8_linear(x.float().numpy(), w.numpy(), we.numpy())
    o = np_(out.float())
    if spread:
        absprod = (np.abs(ref_linear.mx_dequant(info["xq"], info["xe"]))
                   @ np.abs(ref_linear.mx_dequant(w.numpy(), we.numpy())).T)
        d = np.abs(o - ref)
        over = d - (1e-2 + 2e-2 * np.abs(ref) + MX_MFMA_ERR * absprod)
        assert np.isfinite(o).all() and over.max() <= 0, f"{what}: {int((over > 0).sum())} outputs off"
        rel = float(np.linalg.norm(o - ref) / np.linalg.norm(ref))
        assert rel < 1e-2, f"{what}: relative norm error {rel}"
        note(f"  max|d|={d.max():.3e} rel_norm={rel:.3e}")
        return
    m = assert_out_close(o, ref, what)
    note(f"  max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e}")


@pytest.mark.parametrize("M,N,K", [
    (1, 128, 256),      # one row, K split in two slices
    (5, 256, 384),      # ragged block, three K blocks (no split)
    (17, 128, 1024),
    (64, 256, 1152),    # nine K blocks
    (100, 1024, 512),   # K split in two slices
    (300, 640, 256),    # N not a multiple of 256, two K blocks
    (130, 256, 2048),   # two row blocks, K split
    (4096, 4096, 1024), # 512 tiles: two per persistent workgroup
])
@pytest.mark.parametrize("kind", ["synth", "spread"])
def test_mx_linear_small(M, N, K, kind):
    note(f"mxfp8 linear {kind} M={M} N={N} K={K}")
    if kind == "synth":
        x, w, we = make_mx_linear(M, N, K, seed_base=M + N + K)
    else:
        x, w, we = _mx_spread(M, N, K, seed=M * 3 + N + K)
    _mx_check(x, w, we, f"mxfp8 linear {kind} {M}x{N}x{K}", spread=kind == "spread")


@pytest.mark.parametrize("M", [5, 300])
def test_mx_linear_workspace_contents_do_not_matter(M):
    N, K = 640, 256
    x, w, we = make_mx_linear(M, N, K, seed_base=78)
    xd, wd, wed = x.cuda(), w.cuda(), we.cuda()
    n = moe.mxfp8_linear_workspace_bytes(M, N, K)
    clean = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dirty = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN codes and NaN exponents
    note("mxfp8 linear workspace garbage")
    a = moe.mxfp8_linear(xd, wd, wed, workspace=clean)
    b = moe.mxfp8_linear(xd, wd, wed, workspace=dirty)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.isfinite(a.float()).all()


@pytest.mark.parametrize("M", MX_LINEAR_WORKLOAD["M"])
def test_mx_linear_full_size(M):
    N, K = MX_LINEAR_WORKLOAD["N"], MX_LINEAR_WORKLOAD["K"]
    x, w, we = make_mx_linear(M, N, K, 1000 * MX_LINEAR_WORKLOAD["index"], device="cuda")
    note(f"mxfp8 linear full-size M={M} N={N} K={K}")
    out = moe.mxfp8_linear(x, w, we)
    torch.cuda.synchronize()
    rows = _rows(M, M + 1)
    ref, _ = ref_linear.mxfp8_linear(np_(x[torch.from_numpy(rows).cuda()].float()), np_(w), np_(we))
    m = assert_out_close(np_(out.float())[rows], ref, f"mxfp8 linear full-size M={M}")
    note(f"  {rows.size} rows: max|d|={m['max_abs']:.3e} rel_norm={m['rel_norm']:.3e}")
