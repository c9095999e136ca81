"""Host-side pieces of bench.py: the algorithmic byte / flop counts the
roofline uses, the bound selection, and the one-GPU guard."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_counts_by_hand():
    # 3 tokens, top-2 over 4 experts; experts 0, 2 and 3 are used, 1 is not
    T, H, I, E, k = 3, 256, 128, 4, 2
    ids = np.array([[0, 2], [2, 3], [0, 3]])
    a = bench.algorithmic(ids, T, H, I, E, k)
    P = T * k
    w13 = 2 * I * H + 4 * (2 * I // 128) * (H // 128)     # codes + float32 block scales
    w2 = H * I + 4 * (H // 128) * (I // 128)
    assert a["active_experts"] == 3
    assert a["layer_bytes"] == 3 * (w13 + w2) + 2 * T * H + 2 * T * H + 4 * T * E
    assert a["layer_flops"] == 6 * P * H * I
    assert a["stage"]["gemm1"][1] == 4 * P * H * I and a["stage"]["gemm2"][1] == 2 * P * H * I
    # the stages' flops add up to the layer's
    assert sum(f for _, f in a["stage"].values()) == a["layer_flops"]


def test_roofline_bound_selection():
    # 1 GB and 1 TFLOP in 1 ms: 1 TB/s of 8, 1 PFLOP/s of 5 -> the HBM time
    # (0.125 ms) is below the MFMA time (0.2 ms), so MFMA-bound
    r = bench.roofline_of(1e9, 1e12, 1e-3)
    assert r["bound"] == "mfma" and abs(r["achieved"] - 1000.0) < 1e-9 and abs(r["frac"] - 0.2) < 1e-12
    r = bench.roofline_of(4e9, 1e9, 1e-3)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and abs(r["frac"] - 0.5) < 1e-12
    # against the f16 peak the same flops are twice the fraction
    r = bench.roofline_of(1e9, 1e12, 1e-3, bench.MFMA_F16_PEAK)
    assert abs(r["frac"] - 0.4) < 1e-12


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_roofline_at_a_given_bound():
    r = bench.roofline_at(1e9, 1e12, 1e-3, "mfma")
    assert r["peak"] == 5000.0 and abs(r["frac"] - 0.2) < 1e-12
    r = bench.roofline_at(4e9, 1e12, 1e-3, "hbm")
    assert r["unit"] == "GB/s" and abs(r["frac"] - 0.5) < 1e-12


def test_fractions_take_the_larger_of_the_two_bounds():
    f = bench.fractions(4e9, 1e12, 1e-3)          # 0.5 of HBM, 0.2 of FP8 MFMA
    assert abs(f["hbm_frac"] - 0.5) < 1e-12 and abs(f["mfma_frac"] - 0.2) < 1e-12
    assert abs(f["roofline_frac"] - 0.5) < 1e-12 and f["bound_at_peak"] == "hbm"
    assert bench.fractions(1e9, 1e12, 1e-3)["bound_at_peak"] == "mfma"


def test_stats_median_and_percentiles():
    s = bench.stats([float(i) for i in range(1, 12)])     # 1 .. 11
    assert s["median_ms"] == 6.0 and s["n"] == 11
    assert abs(s["p10_ms"] - 2.0) < 1e-12 and abs(s["p90_ms"] - 10.0) < 1e-12


def test_dominant_kernel_bound_follows_its_phase():
    kernels = {"prefill.gemm1": {"ms": 4.0, "bytes": 8e9, "flops": 4e12, "phase": "prefill"},
               "decode.gemm1": {"ms": 1.0, "bytes": 5e9, "flops": 1e10, "phase": "decode"}}
    r = bench.dominant_roofline(kernels, "tiny", None)
    # prefill: against the dense-FP8 peak even though the bytes take longer at peak
    assert r["kernel"] == "prefill.gemm1" and r["bound"] == "mfma" and r["peak"] == 5000.0
    assert abs(r["frac"] - 0.2) < 1e-12 and abs(r["frac_of_f16_peak"] - 0.4) < 1e-12
    assert r["traffic"] is None
    kernels["decode.gemm1"]["ms"] = 5.0
    r = bench.dominant_roofline(kernels, "tiny", {"hbm_read_GB_per_s": 6000.0})
    assert r["bound"] == "hbm" and abs(r["achieved"] - 1000.0) < 1e-9
    assert abs(r["frac_of_measured_peak"] - 1000.0 / 6000.0) < 1e-12


def test_sections_and_cpu_threads():
    a = bench.parse(["--sections", "layer,peaks"])
    assert a.sections == ["layer", "peaks"]
    assert bench.parse(["--layer-only"]).sections == ["layer"]
    assert bench.parse([]).sections == bench.SECTIONS
    n = bench.cpu_threads()
    assert 1 <= n <= len(os.sched_getaffinity(0))


def test_kernel_code_digest_ignores_comments_only(tmp_path):
    """The per-launch traffic figures stay valid across comment edits of the
    kernel source and lapse with any code edit."""
    src = "int f(int a) {  // add one\n  return a + 1;\n}\n"
    a = tmp_path / "a.hip"
    a.write_text(src)
    b = tmp_path / "b.hip"
    b.write_text("// a header comment\nint f(int a) {   \n\n  return a + 1;  // the same\n}\n")
    c = tmp_path / "c.hip"
    c.write_text(src.replace("+ 1", "+ 2"))
    d = tmp_path / "d.hip"
    d.write_text('const char* s = "a // b";\n')
    e = tmp_path / "e.hip"
    e.write_text('const char* s = "a // c";\n')
    assert bench.kernel_code_digest(str(a)) == bench.kernel_code_digest(str(b))
    assert bench.kernel_code_digest(str(a)) != bench.kernel_code_digest(str(c))
    assert bench.kernel_code_digest(str(d)) != bench.kernel_code_digest(str(e))
