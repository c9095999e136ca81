"""Helpers for the GPU parity tests (compare the HIP path with the oracle)."""

import sys

import numpy as np
import torch

OUT_RTOL = 2e-2      # bf16 layer output: |gpu - ref| <= OUT_ATOL + OUT_RTOL * |ref|
OUT_ATOL = 1e-2
OUT_REL_NORM = 1e-2  # and ||gpu - ref|| / ||ref|| below this (see the test docstrings)
WEIGHT_RTOL = 1e-5   # routing weights: device expf vs float64 softmax


def note(msg):
    """Name the case before a GPU step, flushed, so a failing run says where."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(w, dev="cuda"):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}


def np_(t):
    return t.detach().cpu().numpy()


def out_metrics(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(gpu - ref)
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "viol": int(np.sum(d > OUT_ATOL + OUT_RTOL * np.abs(ref))),
        "rel_norm": float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)),
        "finite": bool(np.all(np.isfinite(gpu))),
    }


def assert_out_close(gpu, ref, what=""):
    m = out_metrics(gpu, ref)
    assert m["finite"], f"{what}: non-finite output"
    assert m["viol"] == 0, f"{what}: {m['viol']} outputs outside tolerance, max |d| {m['max_abs']}"
    assert m["rel_norm"] < OUT_REL_NORM, f"{what}: relative norm error {m['rel_norm']}"
    return m


def align_prefix(sorted_ids, expert_ids, ntpp, bm):
    n = int(np_(ntpp)[0])
    return np_(sorted_ids)[:n], np_(expert_ids)[: n // bm], n
