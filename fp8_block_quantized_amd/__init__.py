"""Python binding of libmoe_fp8.so, the gfx950 fused FP8 block-quantized MoE
library.  Argument marshalling only: every step of the computation runs in
the HIP kernels behind the C ABI declared in include/moe_fp8.h.  torch is
used for device memory and streams.  There is no fallback: if the shared
library is missing or a tensor is not a contiguous GPU tensor of the right
type, the call raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_fp8.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_UNSUPPORTED",
          -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_HIP", -6: "MOE_ERR_ALIAS", -7: "MOE_ERR_SCRATCH"}
TAPS = ["topk_ids", "topk_weights", "sorted_ids", "expert_ids", "ntpp", "pair_pos", "xq", "xs",
        "aq", "as", "y", "align_scratch", "y_slices", "h_slices"]
MAX_EXPERTS = 512
MAX_TOKENS = 16384
MAX_TOP_K = 32
QUANT_GROUP = 128

STAGES = ["router", "align", "quant", "gemm1", "gemm2", "combine"]

EXPORTS = ["moe_fp8_block_m", "moe_fp8_workspace_bytes", "moe_fp8_workspace_layout",
           "moe_fp8_forward", "moe_fp8_forward_traced", "per_token_group_quant_fp8",
           "per_token_group_quant_fp8_fmt", "moe_topk_softmax", "moe_topk_softmax_grouped",
           "moe_fp8_forward_routed", "moe_fp8_batched_workspace_bytes", "moe_fp8_batched_experts",
           "moe_fp8_mx_workspace_bytes", "moe_fp8_mx_workspace_layout", "moe_fp8_mx_forward",
           "moe_align_scratch_bytes", "moe_align", "moe_align_noalloc",
           "moe_align_noalloc_max_scratch_bytes", "moe_status_string",
           "fp8_block_linear_workspace_bytes", "fp8_block_linear",
           "mxfp8_linear_workspace_bytes", "mxfp8_linear", "moe_mfma_rate_probe",
           "moe_hbm_read_probe"]


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


_lib = None


def load_library(path=LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    lib.moe_fp8_block_m.argtypes = [c_int] * 5
    lib.moe_fp8_block_m.restype = c_int
    lib.moe_fp8_workspace_bytes.argtypes = [c_int] * 5
    lib.moe_fp8_workspace_bytes.restype = c_size
    lib.moe_fp8_workspace_layout.argtypes = [c_int] * 5 + [ctypes.POINTER(c_size)]
    lib.moe_fp8_workspace_layout.restype = c_int
    lib.moe_fp8_forward.argtypes = [vp] * 6 + [c_int] * 6 + [vp, vp, c_size, vp]
    lib.moe_fp8_forward.restype = c_int
    lib.moe_fp8_forward_traced.argtypes = [vp] * 6 + [c_int] * 6 + [vp, vp, c_size, vp,
                                                                   ctypes.POINTER(vp)]
    lib.moe_fp8_forward_traced.restype = c_int
    lib.per_token_group_quant_fp8.argtypes = [vp, c_int, c_int, c_int, vp, vp, vp]
    lib.per_token_group_quant_fp8.restype = c_int
    lib.per_token_group_quant_fp8_fmt.argtypes = [vp, c_int, c_int, c_int, c_int, vp, vp, vp]
    lib.per_token_group_quant_fp8_fmt.restype = c_int
    lib.moe_topk_softmax.argtypes = [vp, c_int, c_int, c_int, c_int, vp, vp, vp]
    lib.moe_topk_softmax.restype = c_int
    lib.moe_topk_softmax_grouped.argtypes = [vp] + [c_int] * 6 + [vp, vp, vp]
    lib.moe_topk_softmax_grouped.restype = c_int
    lib.moe_fp8_forward_routed.argtypes = [vp] * 6 + [c_int] * 8 + [vp, c_int, vp, vp, c_size, vp]
    lib.moe_fp8_forward_routed.restype = c_int
    lib.moe_fp8_batched_workspace_bytes.argtypes = [c_int] * 4
    lib.moe_fp8_batched_workspace_bytes.restype = c_size
    lib.moe_fp8_batched_experts.argtypes = [vp] * 6 + [c_int] * 4 + [vp, vp, c_size, vp]
    lib.moe_fp8_batched_experts.restype = c_int
    lib.moe_fp8_mx_workspace_bytes.argtypes = [c_int] * 5
    lib.moe_fp8_mx_workspace_bytes.restype = c_size
    lib.moe_fp8_mx_workspace_layout.argtypes = [c_int] * 5 + [ctypes.POINTER(c_size)]
    lib.moe_fp8_mx_workspace_layout.restype = c_int
    lib.moe_fp8_mx_forward.argtypes = [vp] * 6 + [c_int] * 6 + [vp, vp, c_size, vp]
    lib.moe_fp8_mx_forward.restype = c_int
    lib.moe_align_scratch_bytes.argtypes = [c_int] * 3
    lib.moe_align_scratch_bytes.restype = c_size
    lib.moe_align.argtypes = [vp, c_int, c_int, c_int, c_int, vp, vp, vp, vp, c_size, vp]
    lib.moe_align.restype = c_int
    lib.moe_align_noalloc.argtypes = [vp, c_int, c_int, c_int, c_int, vp, vp, vp, vp]
    lib.moe_align_noalloc.restype = c_int
    lib.moe_align_noalloc_max_scratch_bytes.argtypes = []
    lib.moe_align_noalloc_max_scratch_bytes.restype = c_size
    lib.fp8_block_linear_workspace_bytes.argtypes = [c_int] * 3
    lib.fp8_block_linear_workspace_bytes.restype = c_size
    lib.fp8_block_linear.argtypes = [vp, vp, vp, c_int, c_int, c_int, vp, vp, c_size, vp]
    lib.fp8_block_linear.restype = c_int
    lib.mxfp8_linear_workspace_bytes.argtypes = [c_int] * 3
    lib.mxfp8_linear_workspace_bytes.restype = c_size
    lib.mxfp8_linear.argtypes = [vp, vp, vp, c_int, c_int, c_int, vp, vp, c_size, vp]
    lib.mxfp8_linear.restype = c_int
    lib.moe_status_string.argtypes = [c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_mfma_rate_probe.argtypes = [c_int, c_int, c_int, vp, vp]
    lib.moe_mfma_rate_probe.restype = c_int
    lib.moe_hbm_read_probe.argtypes = [vp, c_size, c_int, vp, vp]
    lib.moe_hbm_read_probe.restype = c_int
    _lib = lib
    return lib


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, want, name):
    """Raise ValueError unless tensor t has exactly the shape want (checked
    before anything reaches the library, so a mismatched tensor never lets a
    kernel read or write past an allocation)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} must have shape {tuple(want)}, got {tuple(t.shape)}")


def _ndim(t, n, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _same_device(ref, named):
    for name, t in named.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, x on {ref.device}")


def _multiple(v, m, name):
    if v % m:
        raise ValueError(f"{name} = {v} must be a multiple of {m}")


def _check_moe_tensors(x, router_logits, w13, w13_scale, w2, w2_scale, out, mx=False,
                       all_experts=True):
    """Full shape and device checks of a fused-MoE call; returns (T, H, I, E, EL).
    EL is the expert count of the weights, which must be E when all_experts."""
    T, H = _ndim(x, 2, "x")
    T2, E = _ndim(router_logits, 2, "router_logits")
    if T2 != T:
        raise ValueError(f"router_logits has {T2} rows, x has {T}")
    EL, N13, H13 = _ndim(w13, 3, "w13")
    EL2, H2, I = _ndim(w2, 3, "w2")
    if EL2 != EL:
        raise ValueError(f"w2 holds {EL2} experts, w13 {EL}")
    if all_experts and EL != E:
        raise ValueError(f"the weights hold {EL} experts, the router logits {E}")
    _multiple(H, QUANT_GROUP, "hidden size")
    _multiple(I, QUANT_GROUP, "intermediate size")
    _shape(w13, (EL, 2 * I, H), "w13")
    _shape(w2, (EL, H, I), "w2")
    if mx:
        _shape(w13_scale, (EL, 2 * I, H // 32), "w13_scale")
        _shape(w2_scale, (EL, H, I // 32), "w2_scale")
    else:
        _shape(w13_scale, (EL, 2 * I // 128, H // 128), "w13_scale")
        _shape(w2_scale, (EL, H // 128, I // 128), "w2_scale")
    if out is not None:
        _shape(out, (T, H), "out")
    _same_device(x, {"router_logits": router_logits, "w13": w13, "w13_scale": w13_scale,
                     "w2": w2, "w2_scale": w2_scale, "out": out})
    return T, H, I, E, EL


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moe_fp8_block_m(T, H, I, E, top_k):
    r = load_library().moe_fp8_block_m(T, H, I, E, top_k)
    _check("moe_fp8_block_m", r if r < 0 else 0)
    return r


def moe_fp8_workspace_bytes(T, H, I, E, top_k):
    return load_library().moe_fp8_workspace_bytes(T, H, I, E, top_k)


def moe_fp8_workspace_layout(T, H, I, E, top_k, mx=False):
    offs = (ctypes.c_size_t * len(TAPS))()
    fn = "moe_fp8_mx_workspace_layout" if mx else "moe_fp8_workspace_layout"
    _check(fn, getattr(load_library(), fn)(T, H, I, E, top_k, offs))
    return dict(zip(TAPS, list(offs)))


def alloc_workspace(T, H, I, E, top_k, device="cuda"):
    n = moe_fp8_workspace_bytes(T, H, I, E, top_k)
    if n == 0:
        raise MoeError("moe_fp8_workspace_bytes", -2)
    return torch.empty(n, dtype=torch.uint8, device=device)   # caching allocator: 512-B aligned


def moe_fp8_forward(x, router_logits, w13, w13_scale, w2, w2_scale, top_k, renormalize,
                    out=None, workspace=None, stream=None, events=None):
    """Fused FP8 MoE forward.  x bf16 [T, H], router_logits f32 [T, E],
    w13 uint8 [E, 2I, H], w13_scale f32 [E, 2I/128, H/128], w2 uint8 [E, H, I],
    w2_scale f32 [E, H/128, I/128].  Returns out bf16 [T, H].
    With ``events`` (len(STAGES) + 1 timing-enabled torch.cuda.Event objects
    that have been recorded once), calls moe_fp8_forward_traced, which records
    them around each stage on the launch stream."""
    T, H, I, E, _ = _check_moe_tensors(x, router_logits, w13, w13_scale, w2, w2_scale, out)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, top_k, x.device)
    args = [_dev(x, torch.bfloat16, "x"), _dev(router_logits, torch.float32, "router_logits"),
            _dev(w13, torch.uint8, "w13"), _dev(w13_scale, torch.float32, "w13_scale"),
            _dev(w2, torch.uint8, "w2"), _dev(w2_scale, torch.float32, "w2_scale"),
            T, H, I, E, int(top_k), int(bool(renormalize)),
            _dev(out, torch.bfloat16, "out"), _dev(workspace, torch.uint8, "workspace"),
            workspace.numel(), _stream(stream)]
    lib = load_library()
    if events is None:
        _check("moe_fp8_forward", lib.moe_fp8_forward(*args))
    else:
        if len(events) != len(STAGES) + 1:
            raise ValueError(f"need {len(STAGES) + 1} events")
        handles = (ctypes.c_void_p * len(events))(*[ev.cuda_event for ev in events])
        _check("moe_fp8_forward_traced", lib.moe_fp8_forward_traced(*args, handles))
    return out


def moe_fp8_forward_routed(x, router_logits, w13, w13_scale, w2, w2_scale, top_k, renormalize,
                           num_expert_group=1, topk_group=1, expert_map=None, out=None,
                           workspace=None, stream=None):
    """moe_fp8_forward with grouped top-k and/or an expert map (int32 [E] on the
    device, global -> local expert or -1); the weights hold the local experts."""
    T, H, I, E, EL = _check_moe_tensors(x, router_logits, w13, w13_scale, w2, w2_scale, out,
                                        all_experts=expert_map is None)
    if expert_map is not None:
        _shape(expert_map, (E,), "expert_map")
        _same_device(x, {"expert_map": expert_map})
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, top_k, x.device)
    emap = None if expert_map is None else _dev(expert_map, torch.int32, "expert_map")
    st = load_library().moe_fp8_forward_routed(
        _dev(x, torch.bfloat16, "x"), _dev(router_logits, torch.float32, "router_logits"),
        _dev(w13, torch.uint8, "w13"), _dev(w13_scale, torch.float32, "w13_scale"),
        _dev(w2, torch.uint8, "w2"), _dev(w2_scale, torch.float32, "w2_scale"),
        T, H, I, E, int(top_k), int(bool(renormalize)), int(num_expert_group), int(topk_group),
        emap, EL, _dev(out, torch.bfloat16, "out"), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream))
    _check("moe_fp8_forward_routed", st)
    return out


def workspace_taps(workspace, T, H, I, E, top_k, mx=False):
    """Views of the forward's intermediates inside its workspace (mx: the
    MXFP8 layer's, with exponent bytes in xs / as)."""
    off = moe_fp8_workspace_layout(T, H, I, E, top_k, mx)
    bm = moe_fp8_block_m(T, H, I, E, top_k)
    P = T * top_k
    cap = -(-(P + E * (bm - 1)) // bm) * bm
    ys = -(-H // 256) * 256
    total = (moe_fp8_mx_workspace_bytes if mx else moe_fp8_workspace_bytes)(T, H, I, E, top_k)
    # the two last regions: the GEMMs' K-slice partials (empty without slices)
    nslices = (off["h_slices"] - off["y_slices"]) // (4 * P * ys)
    nslices1 = (total - off["h_slices"]) // (8 * P * 2 * I)
    if workspace.numel() < total:
        nslices = nslices1 = 0          # a batched-format workspace: no K-slice regions

    def view(name, dtype, shape):
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return workspace[off[name]:off[name] + nbytes].view(dtype).view(shape)

    return {
        "block_m": bm, "cap": cap,
        "topk_ids": view("topk_ids", torch.int32, (T, top_k)),
        "topk_weights": view("topk_weights", torch.float32, (T, top_k)),
        "sorted_ids": view("sorted_ids", torch.int32, (cap,)),
        "expert_ids": view("expert_ids", torch.int32, (cap // bm,)),
        "ntpp": view("ntpp", torch.int32, (1,)),
        "pair_pos": view("pair_pos", torch.int32, (P,)),
        "xq": view("xq", torch.uint8, (T, H)),
        "xs": view("xs", torch.uint8, (T, H // 32)) if mx else view("xs", torch.float32, (T, H // 128)),
        "aq": view("aq", torch.uint8, (cap, I)),
        "as": view("as", torch.uint8, (cap, I // 32)) if mx else view("as", torch.float32, (cap, I // 128)),
        "y": view("y", torch.bfloat16, (cap, -(-H // 256) * 256)),
        "y_slices": (view("y_slices", torch.float32, (nslices, P, ys)) if nslices > 1 else None),
        "h_slices": (view("h_slices", torch.float64, (nslices1, P, 2 * I)) if nslices1 > 1 else None),
    }


def per_token_group_quant_fp8(x, group_size=128, q=None, scales=None, stream=None):
    """x bf16 [M, K] -> (q uint8 e4m3fn codes [M, K], scales f32 [M, K/group])."""
    M, K = _ndim(x, 2, "x")
    if group_size != QUANT_GROUP:
        raise ValueError(f"group_size must be {QUANT_GROUP}")
    _multiple(K, group_size, "K")
    if q is not None:
        _shape(q, (M, K), "q")
    if scales is not None:
        _shape(scales, (M, K // group_size), "scales")
    _same_device(x, {"q": q, "scales": scales})
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // group_size), dtype=torch.float32, device=x.device)
    st = load_library().per_token_group_quant_fp8(
        _dev(x, torch.bfloat16, "x"), M, K, group_size, _dev(q, torch.uint8, "q"),
        _dev(scales, torch.float32, "scales"), _stream(stream))
    _check("per_token_group_quant_fp8", st)
    return q, scales


SCALE_FORMATS = {"float32": 0, "float32_ceil_ue8m0": 1, "ue8m0": 2}


def per_token_group_quant_fp8_fmt(x, group_size=128, scale_format="float32", q=None, scales=None,
                                  stream=None):
    """x bf16 [M, K] -> (q uint8 e4m3fn codes [M, K], scales [M, K/group]): float32
    scales for "float32" and "float32_ceil_ue8m0", uint8 exponent bytes for "ue8m0"."""
    M, K = _ndim(x, 2, "x")
    if group_size not in (32, 128):
        raise ValueError("group_size must be 32 or 128")
    _multiple(K, group_size, "K")
    if scale_format not in SCALE_FORMATS:
        raise ValueError(f"scale_format must be one of {sorted(SCALE_FORMATS)}")
    if q is not None:
        _shape(q, (M, K), "q")
    if scales is not None:
        _shape(scales, (M, K // group_size), "scales")
    _same_device(x, {"q": q, "scales": scales})
    fmt = SCALE_FORMATS[scale_format]
    sdt = torch.uint8 if scale_format == "ue8m0" else torch.float32
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // group_size), dtype=sdt, device=x.device)
    st = load_library().per_token_group_quant_fp8_fmt(
        _dev(x, torch.bfloat16, "x"), M, K, group_size, fmt, _dev(q, torch.uint8, "q"),
        _dev(scales, sdt, "scales"), _stream(stream))
    _check("per_token_group_quant_fp8_fmt", st)
    return q, scales


def moe_topk_softmax(logits, top_k, renormalize, ids=None, weights=None, stream=None):
    """logits f32 [T, E] -> (ids int32 [T, k], weights f32 [T, k])."""
    T, E = _ndim(logits, 2, "logits")
    for name, t in (("ids", ids), ("weights", weights)):
        if t is not None:
            _shape(t, (T, top_k), name)
    _same_device(logits, {"ids": ids, "weights": weights})
    if ids is None:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    st = load_library().moe_topk_softmax(
        _dev(logits, torch.float32, "logits"), T, E, int(top_k), int(bool(renormalize)),
        _dev(ids, torch.int32, "ids"), _dev(weights, torch.float32, "weights"), _stream(stream))
    _check("moe_topk_softmax", st)
    return ids, weights


def moe_topk_softmax_grouped(logits, top_k, num_expert_group, topk_group, renormalize, ids=None,
                             weights=None, stream=None):
    """Grouped top-k: logits f32 [T, E] -> (ids int32 [T, k], weights f32 [T, k])."""
    T, E = _ndim(logits, 2, "logits")
    for name, t in (("ids", ids), ("weights", weights)):
        if t is not None:
            _shape(t, (T, top_k), name)
    _same_device(logits, {"ids": ids, "weights": weights})
    if ids is None:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    st = load_library().moe_topk_softmax_grouped(
        _dev(logits, torch.float32, "logits"), T, E, int(top_k), int(num_expert_group),
        int(topk_group), int(bool(renormalize)), _dev(ids, torch.int32, "ids"),
        _dev(weights, torch.float32, "weights"), _stream(stream))
    _check("moe_topk_softmax_grouped", st)
    return ids, weights


def moe_align(topk_ids, num_experts, block_m, stream=None):
    """topk_ids int32 [T, k] -> (sorted_ids, expert_ids, num_tokens_post_padded)
    over the full capacity; only the first num_tokens_post_padded rows are defined."""
    T, k = _ndim(topk_ids, 2, "topk_ids")
    P = T * k
    cap = -(-(P + num_experts * (block_m - 1)) // block_m) * block_m
    dev = topk_ids.device
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    expert_ids = torch.empty(cap // block_m, dtype=torch.int32, device=dev)
    ntpp = torch.empty(1, dtype=torch.int32, device=dev)
    lib = load_library()
    nscr = lib.moe_align_scratch_bytes(T, k, num_experts)
    scratch = torch.empty(max(nscr, 4), dtype=torch.uint8, device=dev)
    st = lib.moe_align(_dev(topk_ids, torch.int32, "topk_ids"), T, k, num_experts, block_m,
                       _dev(sorted_ids, torch.int32, "sorted_ids"),
                       _dev(expert_ids, torch.int32, "expert_ids"), _dev(ntpp, torch.int32, "ntpp"),
                       _dev(scratch, torch.uint8, "scratch"), scratch.numel(), _stream(stream))
    _check("moe_align", st)
    return sorted_ids, expert_ids, ntpp


def moe_align_noalloc(topk_ids, num_experts, block_m, sorted_ids=None, expert_ids=None,
                      ntpp=None, stream=None):
    """moe_align with the library's fixed per-GPU scratch instead of a scratch
    tensor: the call itself allocates no device memory.  Output tensors
    (sorted_ids int32 [cap], expert_ids int32 [cap / block_m], ntpp int32 [1])
    may be passed in to keep the call allocation-free on the Python side too."""
    T, k = _ndim(topk_ids, 2, "topk_ids")
    P = T * k
    cap = -(-(P + num_experts * (block_m - 1)) // block_m) * block_m
    dev = topk_ids.device
    if sorted_ids is None:
        sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(cap // block_m, dtype=torch.int32, device=dev)
    if ntpp is None:
        ntpp = torch.empty(1, dtype=torch.int32, device=dev)
    _shape(sorted_ids, (cap,), "sorted_ids")
    _shape(expert_ids, (cap // block_m,), "expert_ids")
    _shape(ntpp, (1,), "ntpp")
    _same_device(topk_ids, {"sorted_ids": sorted_ids, "expert_ids": expert_ids, "ntpp": ntpp})
    st = load_library().moe_align_noalloc(
        _dev(topk_ids, torch.int32, "topk_ids"), T, k, num_experts, block_m,
        _dev(sorted_ids, torch.int32, "sorted_ids"), _dev(expert_ids, torch.int32, "expert_ids"),
        _dev(ntpp, torch.int32, "ntpp"), _stream(stream))
    _check("moe_align_noalloc", st)
    return sorted_ids, expert_ids, ntpp


def fp8_block_linear_workspace_bytes(M, N, K):
    return load_library().fp8_block_linear_workspace_bytes(M, N, K)


def fp8_block_linear(x, w, w_scale, out=None, workspace=None, stream=None):
    """Dense block-FP8 linear: x bf16 [M, K], w uint8 e4m3fn [N, K], w_scale f32
    [N/128, K/128] -> out bf16 [M, N] (x quantised per 128-group of each row)."""
    M, K = _ndim(x, 2, "x")
    N, K2 = _ndim(w, 2, "w")
    if K2 != K:
        raise ValueError(f"w has {K2} input features, x has {K}")
    _multiple(N, 128, "N")
    _multiple(K, 128, "K")
    _shape(w_scale, (N // 128, K // 128), "w_scale")
    if out is not None:
        _shape(out, (M, N), "out")
    _same_device(x, {"w": w, "w_scale": w_scale, "out": out})
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        n = fp8_block_linear_workspace_bytes(M, N, K)
        if n == 0:
            raise MoeError("fp8_block_linear_workspace_bytes", -2)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    st = load_library().fp8_block_linear(
        _dev(x, torch.bfloat16, "x"), _dev(w, torch.uint8, "w"), _dev(w_scale, torch.float32, "w_scale"),
        M, N, K, _dev(out, torch.bfloat16, "out"), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream))
    _check("fp8_block_linear", st)
    return out


def mxfp8_linear_workspace_bytes(M, N, K):
    return load_library().mxfp8_linear_workspace_bytes(M, N, K)


def mxfp8_linear(x, w, w_scale, out=None, workspace=None, stream=None):
    """MXFP8 dense linear: x bf16 [M, K], w uint8 e4m3fn [N, K], w_scale uint8
    UE8M0 exponents [N, K/32] -> out bf16 [M, N] (x quantised per 32-group of
    each row with power-of-two scales)."""
    M, K = _ndim(x, 2, "x")
    N, K2 = _ndim(w, 2, "w")
    if K2 != K:
        raise ValueError(f"w has {K2} input features, x has {K}")
    _multiple(N, 128, "N")
    _multiple(K, 128, "K")
    _shape(w_scale, (N, K // 32), "w_scale")
    if out is not None:
        _shape(out, (M, N), "out")
    _same_device(x, {"w": w, "w_scale": w_scale, "out": out})
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        n = mxfp8_linear_workspace_bytes(M, N, K)
        if n == 0:
            raise MoeError("mxfp8_linear_workspace_bytes", -2)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    st = load_library().mxfp8_linear(
        _dev(x, torch.bfloat16, "x"), _dev(w, torch.uint8, "w"), _dev(w_scale, torch.uint8, "w_scale"),
        M, N, K, _dev(out, torch.bfloat16, "out"), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream))
    _check("mxfp8_linear", st)
    return out


def moe_fp8_batched_workspace_bytes(E, max_tokens, H, I):
    return load_library().moe_fp8_batched_workspace_bytes(E, max_tokens, H, I)


def moe_fp8_batched_experts(x, expert_num_tokens, w13, w13_scale, w2, w2_scale, out=None,
                            workspace=None, stream=None):
    """Batched (masked) expert format: x bf16 [E, M, H], expert_num_tokens int32
    [E] on the device -> out bf16 [E, M, H] (zero past each count)."""
    E, M, H = _ndim(x, 3, "x")
    _shape(expert_num_tokens, (E,), "expert_num_tokens")
    _ndim(w2, 3, "w2")
    I = w2.shape[2]
    _multiple(H, QUANT_GROUP, "hidden size")
    _multiple(I, QUANT_GROUP, "intermediate size")
    _shape(w13, (E, 2 * I, H), "w13")
    _shape(w13_scale, (E, 2 * I // 128, H // 128), "w13_scale")
    _shape(w2, (E, H, I), "w2")
    _shape(w2_scale, (E, H // 128, I // 128), "w2_scale")
    if out is not None:
        _shape(out, (E, M, H), "out")
    _same_device(x, {"expert_num_tokens": expert_num_tokens, "w13": w13, "w13_scale": w13_scale,
                     "w2": w2, "w2_scale": w2_scale, "out": out})
    if out is None:
        out = torch.empty((E, M, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        n = moe_fp8_batched_workspace_bytes(E, M, H, I)
        if n == 0:
            raise MoeError("moe_fp8_batched_workspace_bytes", -2)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    st = load_library().moe_fp8_batched_experts(
        _dev(x, torch.bfloat16, "x"), _dev(expert_num_tokens, torch.int32, "expert_num_tokens"),
        _dev(w13, torch.uint8, "w13"), _dev(w13_scale, torch.float32, "w13_scale"),
        _dev(w2, torch.uint8, "w2"), _dev(w2_scale, torch.float32, "w2_scale"),
        E, M, H, I, _dev(out, torch.bfloat16, "out"), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream))
    _check("moe_fp8_batched_experts", st)
    return out


def moe_fp8_mx_workspace_bytes(T, H, I, E, top_k):
    return load_library().moe_fp8_mx_workspace_bytes(T, H, I, E, top_k)


def moe_fp8_mx_forward(x, router_logits, w13, w13_scale, w2, w2_scale, top_k, renormalize,
                       out=None, workspace=None, stream=None):
    """MXFP8 MoE forward: w13 uint8 [E, 2I, H] with UE8M0 bytes [E, 2I, H/32],
    w2 uint8 [E, H, I] with UE8M0 bytes [E, H, I/32]."""
    T, H, I, E, _ = _check_moe_tensors(x, router_logits, w13, w13_scale, w2, w2_scale, out,
                                       mx=True)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        n = moe_fp8_mx_workspace_bytes(T, H, I, E, top_k)
        if n == 0:
            raise MoeError("moe_fp8_mx_workspace_bytes", -2)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    st = load_library().moe_fp8_mx_forward(
        _dev(x, torch.bfloat16, "x"), _dev(router_logits, torch.float32, "router_logits"),
        _dev(w13, torch.uint8, "w13"), _dev(w13_scale, torch.uint8, "w13_scale"),
        _dev(w2, torch.uint8, "w2"), _dev(w2_scale, torch.uint8, "w2_scale"),
        T, H, I, E, int(top_k), int(bool(renormalize)), _dev(out, torch.bfloat16, "out"),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check("moe_fp8_mx_forward", st)
    return out


MFMA_PROBE_FLOPS = {"f16": 16384, "fp8": 65536}    # per instruction


def moe_mfma_rate_probe(kind, iters, nblocks, sink, stream=None):
    """Matrix-core rate probe ("f16": the first GEMM's v_mfma_f32_16x16x32_f16,
    "fp8": the second GEMM's FP8 16x16x128): nblocks x 4 waves x iters x 8
    MFMAs from registers; sink is a float32 device tensor of nblocks * 256.
    Returns the flops the launch performs."""
    k = {"f16": 0, "fp8": 1}[kind]
    if sink.numel() < nblocks * 256:
        raise ValueError("sink needs nblocks * 256 floats")
    st = load_library().moe_mfma_rate_probe(k, int(iters), int(nblocks),
                                            _dev(sink, torch.float32, "sink"), _stream(stream))
    _check("moe_mfma_rate_probe", st)
    return nblocks * 4 * iters * 8 * MFMA_PROBE_FLOPS[kind]


def moe_hbm_read_probe(src, nblocks, sink, stream=None):
    """HBM read-stream probe: reads the bytes of the contiguous GPU tensor src
    once (its size a multiple of 16 bytes); sink is an int32 device tensor of
    nblocks * 256 that receives one XOR word per thread.  Returns the bytes read."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise TypeError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    if sink.numel() < nblocks * 256:
        raise ValueError("sink needs nblocks * 256 words")
    st = load_library().moe_hbm_read_probe(ctypes.c_void_p(src.data_ptr()), nbytes, int(nblocks),
                                           _dev(sink, torch.int32, "sink"), _stream(stream))
    _check("moe_hbm_read_probe", st)
    return nbytes
