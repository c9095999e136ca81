"""Builds libmoe_fp8.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc."""

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_fp8.so")
ARCH = "gfx950"

SOURCES = ["moe_fp8.cpp", "quant.hip", "router.hip", "align.hip", "front.hip", "gemm.hip", "combine.hip",
           "probe.hip"]

# -ffp-contract=off: the arithmetic is exactly as written (explicit fmaf where
# a fused multiply-add is wanted).  Packed fp32 VALU ops are disabled.
# -amdgpu-mfma-vgpr-form: MFMA accumulators in ordinary VGPRs; otherwise the
# register allocator may park them in AGPRs and copy them back and forth
# around every MFMA inside a loop (in the decode GEMMs, and in a register-only
# MFMA loop, where the copies halved the f16 rate).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wno-unused-command-line-argument"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + HIP_FLAGS + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj, r.stderr


def build(extra_flags=(), verbose=False) -> str:
    """Compile every HIP source for gfx950 and link libmoe_fp8.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    if verbose:
        for _, err in results:
            if err.strip():
                print(err)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
