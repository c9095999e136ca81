"""CPU tests of the C ABI: the library loads, exports every function that
include/moe_fp8.h declares (and the binding knows them), and its host-side
logic (argument checks, block size, workspace layout) behaves as documented.
No kernel is launched: every call here fails validation before any HIP call,
or is pure host arithmetic."""

import ctypes
import os
import re
import subprocess

import pytest

import fp8_block_quantized_amd as moe

HDR = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_fp8.h")


def _declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True)
    for name in _declared():
        assert re.search(rf" T {name}$", nm.stdout, flags=re.M), name


def test_status_strings():
    lib = moe.load_library()
    for code in range(-7, 1):
        assert lib.moe_status_string(code)
    assert lib.moe_status_string(7) == b"unknown status"


@pytest.mark.parametrize("T,H,I,E,k,bad", [
    (0, 256, 256, 8, 2, True), (16, 200, 256, 8, 2, True), (16, 256, 100, 8, 2, True),
    (16, 256, 256, 0, 1, True), (16, 256, 256, 8, 9, True), (16, 256, 256, 513, 2, True),
    (16385, 256, 256, 8, 2, True), (16, 256, 256, 64, 33, True), (16, 256, 256, 8, 0, True),
    (16, 256, 256, 8, 2, False), (16384, 7168, 2048, 512, 32, False)])
def test_shape_checks(T, H, I, E, k, bad):
    ws = moe.moe_fp8_workspace_bytes(T, H, I, E, k)
    bm = moe.load_library().moe_fp8_block_m(T, H, I, E, k)
    if bad:
        assert ws == 0 and bm == -2
    else:
        assert ws > 0 and bm in (16, 32, 64, 128)


def test_block_m_choices():
    bm = lambda *a: moe.moe_fp8_block_m(*a)
    assert bm(64, 7168, 2048, 256, 8) == 16      # decode: ~2 pairs per expert
    assert bm(1, 2048, 768, 128, 8) == 16
    assert bm(64, 4096, 14336, 8, 2) == 32       # 16 pairs per expert
    assert bm(8192, 7168, 2048, 256, 8) == 128   # prefill
    assert bm(4096, 2048, 768, 128, 8) == 128


def test_workspace_layout_is_disjoint_and_aligned():
    for shape in [(16, 256, 512, 8, 2), (64, 7168, 2048, 256, 8), (8192, 7168, 2048, 256, 8),
                  (1, 2048, 768, 128, 8), (512, 4096, 14336, 8, 2), (64, 4096, 14336, 8, 2),
                  (32, 2048, 768, 128, 8)]:
        T, H, I, E, k = shape
        off = moe.moe_fp8_workspace_layout(*shape)
        total = moe.moe_fp8_workspace_bytes(*shape)
        bm = moe.moe_fp8_block_m(*shape)
        P = T * k
        cap = -(-(P + E * (bm - 1)) // bm) * bm
        size = {"topk_ids": 4 * P, "topk_weights": 4 * P, "sorted_ids": 4 * cap,
                "expert_ids": 4 * (cap // bm), "ntpp": 4, "pair_pos": 4 * P, "xq": T * H, "xs": 4 * T * H // 128,
                "aq": cap * I, "as": 4 * cap * I // 128, "y": 2 * cap * (-(-H // 256) * 256), "align_scratch": 0,
                "y_slices": 0}
        names = moe.TAPS
        for a, b in zip(names, names[1:]):
            assert off[a] % 256 == 0
            assert off[a] + size[a] <= off[b]
        # the two last regions hold the GEMMs' K-slice partials, or nothing
        ys = -(-H // 256) * 256
        slices2 = (off["h_slices"] - off["y_slices"]) // (4 * P * ys)
        slices1 = (total - off["h_slices"]) // (8 * P * 2 * I)
        assert off["y_slices"] + 4 * P * ys * slices2 <= off["h_slices"]
        assert off["h_slices"] % 256 == 0 and off["h_slices"] + 8 * P * 2 * I * slices1 <= total
        assert (slices1, slices2) == expect_slices[shape]


# K slices (GEMM1, GEMM2) of the decode GEMMs (0: none).  The tiles in use
# (blocks: one per expert plus ceil(P / block_m), at most the capacity;
# GEMM1 times I / 128 feature groups, GEMM2 times ceil(H / 256) feature
# tiles) are raised towards 512 (GEMM1) and 1024 (GEMM2) workgroups, at most
# 8 slices and one per 128-wide K block.
expect_slices = {(16, 256, 512, 8, 2): (2, 4),       # 10 blocks: capped by H / 128, I / 128
                 (64, 7168, 2048, 256, 8): (0, 0),   # 272 blocks x 16 groups, x 28 tiles
                 (8192, 7168, 2048, 256, 8): (0, 0), # block_m 128
                 (1, 2048, 768, 128, 8): (8, 6),     # 9 blocks: 54 groups, 72 tiles
                 (512, 4096, 14336, 8, 2): (0, 0),   # block_m 128
                 (64, 4096, 14336, 8, 2): (0, 6),    # 12 blocks: 1344 groups; 192 tiles
                 (32, 2048, 768, 128, 8): (0, 0)}    # 136 blocks: 816 groups; 1088 tiles


def test_forward_argument_checks():
    lib = moe.load_library()
    vp = ctypes.c_void_p
    fake = [vp(0x10000 * (i + 1)) for i in range(8)]   # never dereferenced: checks fail first
    T, H, I, E, k = 16, 256, 512, 8, 2
    need = moe.moe_fp8_workspace_bytes(T, H, I, E, k)
    ws = vp(0x7000000000)

    def call(args):
        return lib.moe_fp8_forward(*args)

    base = [fake[0], fake[1], fake[2], fake[3], fake[4], fake[5], T, H, I, E, k, 1,
            vp(0x6000000000), ws, need, None]
    for i in range(6):
        a = list(base)
        a[i] = None
        assert call(a) == -1
    a = list(base); a[12] = None; assert call(a) == -1
    a = list(base); a[13] = None; assert call(a) == -1
    a = list(base); a[7] = 300; assert call(a) == -2
    a = list(base); a[11] = 2; assert call(a) == -2
    a = list(base); a[14] = need - 1; assert call(a) == -4
    a = list(base); a[13] = vp(0x7000000010); assert call(a) == -4          # misaligned
    a = list(base); a[12] = vp(0x7000000000 + 512); assert call(a) == -6    # out inside workspace
    a = list(base); a[12] = vp(fake[0].value + 256); assert call(a) == -6   # out overlaps x
    a = list(base); a[0] = vp(fake[0].value + 2); assert call(a) == -3      # x not 16-byte aligned


def test_stage_argument_checks():
    lib = moe.load_library()
    vp = ctypes.c_void_p
    assert lib.per_token_group_quant_fp8(vp(16), 4, 256, 64, vp(4096), vp(8192), None) == -3
    assert lib.per_token_group_quant_fp8(vp(16), 4, 200, 128, vp(4096), vp(8192), None) == -2
    assert lib.per_token_group_quant_fp8(vp(16), -1, 256, 128, vp(4096), vp(8192), None) == -2
    assert lib.per_token_group_quant_fp8(None, 0, 256, 128, None, None, None) == 0   # empty: no-op
    assert lib.per_token_group_quant_fp8(None, 4, 256, 128, vp(4096), vp(8192), None) == -1
    assert lib.per_token_group_quant_fp8(vp(0x10000), 4, 256, 128, vp(0x10000 + 128), vp(1 << 30), None) == -6
    f = lib.per_token_group_quant_fp8_fmt
    assert f(vp(16), 4, 256, 64, 2, vp(4096), vp(8192), None) == -3           # group 64
    assert f(vp(16), 4, 256, 32, 3, vp(4096), vp(8192), None) == -3           # format 3
    assert f(vp(16), 4, 48, 32, 2, vp(4096), vp(8192), None) == -2            # K % 32
    assert f(vp(16), 4, 160, 128, 1, vp(4096), vp(8192), None) == -2          # K % 128
    assert f(None, 0, 256, 32, 2, None, None, None) == 0                      # empty: no-op
    assert f(vp(16), 4, 256, 32, 2, None, vp(8192), None) == -1
    assert f(vp(16), 4, 256, 32, 1, vp(4096), vp(8194), None) == -3           # float scales misaligned
    assert f(vp(0x10000), 4, 256, 32, 2, vp(1 << 20), vp(0x10000 + 2047), None) == -6  # scales in x
    assert lib.moe_topk_softmax(vp(16), 4, 8, 9, 1, vp(64), vp(128), None) == -2
    assert lib.moe_topk_softmax(vp(16), 4, 600, 2, 1, vp(64), vp(128), None) == -2
    assert lib.moe_topk_softmax(None, 4, 8, 2, 1, vp(64), vp(128), None) == -1
    assert lib.moe_topk_softmax(None, 0, 8, 2, 1, None, None, None) == 0
    n = lib.moe_align_scratch_bytes(64, 8, 256)
    assert n == (2 * 1 * 256 + 257) * 4      # per-chunk counts + bases, expert offsets
    assert lib.moe_align(vp(16), 64, 8, 256, 24, vp(64), vp(128), vp(256), vp(512), n, None) == -2
    assert lib.moe_align(vp(16), 64, 8, 256, 16, vp(64), vp(128), vp(256), vp(512), n - 4, None) == -4
    assert lib.moe_align(None, 64, 8, 256, 16, vp(64), vp(128), vp(256), vp(512), n, None) == -1


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        moe.per_token_group_quant_fp8(torch.zeros((2, 128), dtype=torch.bfloat16),
                                      q=torch.zeros((2, 128), dtype=torch.uint8),
                                      scales=torch.zeros((2, 1)))


def test_linear_workspace_and_argument_checks():
    lib = moe.load_library()
    vp = ctypes.c_void_p
    M, N, K = 64, 256, 512
    need = moe.fp8_block_linear_workspace_bytes(M, N, K)
    assert need > 0
    assert moe.fp8_block_linear_workspace_bytes(M, N + 64, K) == 0      # N % 128
    assert moe.fp8_block_linear_workspace_bytes(0, N, K) == 0
    assert moe.fp8_block_linear_workspace_bytes(M, 65536, 65536) == 0  # N*K >= 2^31
    assert moe.fp8_block_linear_workspace_bytes(2 * M, N, K) >= need
    x, w, s, out = (vp(0x10000 * i) for i in (1, 2, 3, 4))
    ws = vp(0x7000000000)

    def call(*a):
        return lib.fp8_block_linear(*a)

    ok = [x, w, s, M, N, K, out, ws, need, None]
    bad = list(ok); bad[5] = 100
    assert call(*bad) == -2                      # shape
    bad = list(ok); bad[0] = None
    assert call(*bad) == -1                      # null
    bad = list(ok); bad[8] = need - 1
    assert call(*bad) == -4                      # workspace too small
    bad = list(ok); bad[6] = vp(0x10000 + 16)
    assert call(*bad) == -6                      # out overlaps x
    bad = list(ok); bad[7] = vp(0x7000000000 + 8)
    assert call(*bad) == -3                      # workspace misaligned


def test_mx_linear_workspace_and_argument_checks():
    lib = moe.load_library()
    vp = ctypes.c_void_p
    M, N, K = 64, 256, 512
    need = moe.mxfp8_linear_workspace_bytes(M, N, K)
    assert need == moe.fp8_block_linear_workspace_bytes(M, N, K) > 0
    assert moe.mxfp8_linear_workspace_bytes(M, N, 128) == 0             # one K block
    assert moe.mxfp8_linear_workspace_bytes(M, N + 64, K) == 0
    x, w, s, out = (vp(0x10000 * i) for i in (1, 2, 3, 4))
    ws = vp(0x7000000000)
    f = lib.mxfp8_linear
    ok = [x, w, s, M, N, K, out, ws, need, None]
    bad = list(ok); bad[5] = 128
    assert f(*bad) == -3                         # K = 128 unsupported
    bad = list(ok); bad[5] = 200
    assert f(*bad) == -2
    bad = list(ok); bad[2] = None
    assert f(*bad) == -1
    bad = list(ok); bad[8] = need - 1
    assert f(*bad) == -4
    bad = list(ok); bad[2] = vp(0x30002)
    assert f(*bad) == -3                         # exponent bytes not 4-byte aligned
    bad = list(ok); bad[6] = vp(0x30000 + 16)
    assert f(*bad) == -6                         # out overlaps the exponents (N*K/32 bytes)


def test_routing_argument_checks():
    # every call below is invalid, so it returns before anything is launched
    lib = moe.load_library()
    vp = ctypes.c_void_p
    g = lib.moe_topk_softmax_grouped
    assert g(vp(16), 4, 256, 8, 7, 4, 1, vp(64), vp(128), None) == -2     # 7 does not divide 256
    assert g(vp(16), 4, 256, 8, 8, 9, 1, vp(64), vp(128), None) == -2     # topk_group > groups
    assert g(vp(16), 4, 256, 8, 128, 1, 1, vp(64), vp(128), None) == -2   # more than 64 groups
    assert g(vp(16), 4, 256, 8, 64, 1, 1, vp(64), vp(128), None) == -2    # top_k > kept experts (4)
    assert g(vp(16), 4, 256, 8, 1, 2, 1, vp(64), vp(128), None) == -2     # one group needs topk_group 1
    assert g(None, 4, 256, 8, 8, 4, 1, vp(64), vp(128), None) == -1
    assert g(None, 0, 256, 8, 8, 4, 1, None, None, None) == 0             # empty: no-op
    T, H, I, E, k = 4, 256, 256, 16, 2
    n = lib.moe_fp8_workspace_bytes(T, H, I, E, k)
    f = lib.moe_fp8_forward_routed
    base = [vp(0x10000 * (i + 1)) for i in range(6)] + [T, H, I, E, k, 1, 1, 1, vp(0x900000), 8,
                                                         vp(0x100000), vp(0x7000000000), n, None]

    def call(a):
        return f(*a)
    a = list(base); a[15] = 17; assert call(a) == -2        # more local experts than E
    a = list(base); a[15] = 0; assert call(a) == -2
    a = list(base); a[14] = None; assert call(a) == -2      # no map: local count must be E
    a = list(base); a[14] = vp(0x900002); assert call(a) == -3     # map misaligned
    a = list(base); a[14] = vp(0x100000 + 8); assert call(a) == -6   # map inside out
    a = list(base); a[12], a[13] = 4, 5; assert call(a) == -2      # topk_group > num_expert_group
    a = list(base); a[12], a[13] = 8, 1; a[10] = 3; assert call(a) == -2   # top_k 3 > one group of 2


def test_batched_argument_checks():
    # every call below is invalid, so it returns before anything is launched
    lib = moe.load_library()
    vp = ctypes.c_void_p
    # the forward's layout for E * M tokens at top_k 1, without the K-slice region
    off = moe.moe_fp8_workspace_layout(64, 256, 256, 4, 1)
    assert moe.moe_fp8_batched_workspace_bytes(4, 16, 256, 256) == off["y_slices"]
    assert moe.moe_fp8_batched_workspace_bytes(64, 512, 256, 256) == 0          # E * M > 16384
    n = moe.moe_fp8_batched_workspace_bytes(4, 16, 256, 256)
    f = lib.moe_fp8_batched_experts
    base = [vp(0x10000 * (i + 1)) for i in range(6)] + [4, 16, 256, 256, vp(0x900000),
                                                         vp(0x7000000000), n, None]
    a = list(base); a[6] = 0; assert f(*a) == -2
    a = list(base); a[9] = 200; assert f(*a) == -2             # I not a multiple of 128
    a = list(base); a[1] = None; assert f(*a) == -1
    a = list(base); a[12] = n - 1; assert f(*a) == -4
    a = list(base); a[1] = vp(0x20002); assert f(*a) == -3     # counts misaligned
    a = list(base); a[10] = vp(0x10000 + 64); assert f(*a) == -6   # out overlaps x


def test_mx_forward_argument_checks():
    # every call below is invalid, so it returns before anything is launched
    lib = moe.load_library()
    vp = ctypes.c_void_p
    T, H, I, E, k = 4, 256, 256, 8, 2
    n = moe.moe_fp8_mx_workspace_bytes(T, H, I, E, k)
    assert n > 0 and moe.moe_fp8_mx_workspace_bytes(T, H, 128, E, k) == 0     # I < 256
    f = lib.moe_fp8_mx_forward
    base = [vp(0x10000 * (i + 1)) for i in range(6)] + [T, H, I, E, k, 1, vp(0x900000),
                                                         vp(0x7000000000), n, None]
    a = list(base); a[8] = 128; assert f(*a) == -3          # I = 128 unsupported
    a = list(base); a[11] = 2; assert f(*a) == -2           # renormalize not 0/1
    a = list(base); a[3] = None; assert f(*a) == -1
    a = list(base); a[14] = n - 1; assert f(*a) == -4
    a = list(base); a[3] = vp(0x40002); assert f(*a) == -3   # exponents misaligned
    a = list(base); a[12] = vp(0x10000 + 64); assert f(*a) == -6   # out overlaps x


def test_mfma_probe_argument_checks():
    # every call below is invalid, so it returns before anything is launched
    f = moe.load_library().moe_mfma_rate_probe
    vp = ctypes.c_void_p
    sink = vp(0x7000000000)
    assert f(2, 10, 4, sink, None) == -3          # unknown instruction kind
    assert f(0, 0, 4, sink, None) == -2           # no rounds
    assert f(1, 10, 0, sink, None) == -2          # no workgroups
    assert f(0, 10, (1 << 20) + 1, sink, None) == -2
    assert f(0, 10, 4, None, None) == -1          # no sink
    assert f(1, 10, 4, vp(0x7000000002), None) == -3   # misaligned sink
    assert moe.MFMA_PROBE_FLOPS == {"f16": 16 * 16 * 32 * 2, "fp8": 16 * 16 * 128 * 2}


def test_noalloc_align_scratch_limit_and_argument_checks():
    """The scratch-free sort-and-pad: its fixed scratch covers the largest
    request moe_align accepts, and its arguments are checked on the host
    before the device scratch is looked up (no HIP call here)."""
    lib = moe.load_library()
    vp = ctypes.c_void_p
    assert lib.moe_align_noalloc_max_scratch_bytes() == lib.moe_align_scratch_bytes(
        moe.MAX_TOKENS, moe.MAX_TOP_K, moe.MAX_EXPERTS)
    ok = (vp(16), 64, 8, 256, 16, vp(64), vp(128), vp(256), None)
    assert lib.moe_align_noalloc(*ok[:4], 24, *ok[5:]) == -2           # block_m not a power of 2
    assert lib.moe_align_noalloc(ok[0], 64, 8, 513, 16, *ok[5:]) == -2  # too many experts
    assert lib.moe_align_noalloc(ok[0], moe.MAX_TOKENS + 1, moe.MAX_TOP_K, 512, 16, *ok[5:]) == -2
    assert lib.moe_align_noalloc(None, *ok[1:]) == -1
    assert lib.moe_align_noalloc(*ok[:5], None, *ok[6:]) == -1
    assert lib.moe_status_string(-7) != b"unknown status"


def test_hbm_read_probe_argument_checks():
    lib = moe.load_library()
    vp = ctypes.c_void_p
    assert lib.moe_hbm_read_probe(vp(4096), 0, 8, vp(4096), None) == -2
    assert lib.moe_hbm_read_probe(vp(4096), 100, 8, vp(4096), None) == -2
    assert lib.moe_hbm_read_probe(vp(4096), 4096, 0, vp(4096), None) == -2
    assert lib.moe_hbm_read_probe(None, 4096, 8, vp(4096), None) == -1
    assert lib.moe_hbm_read_probe(vp(4100), 4096, 8, vp(4096), None) == -3
