"""Host check of the float32 quotient the quantisation kernels compute (one
multiply by the correctly rounded reciprocal and two FMAs) against IEEE
division: exhaustive over the bf16 activation domain, random over float32
(tests/c/quotient_check.c)."""

import os
import subprocess
import tempfile

import pytest

SRC = os.path.join(os.path.dirname(__file__), "c", "quotient_check.c")


@pytest.fixture(scope="module")
def exe():
    d = tempfile.mkdtemp()
    out = os.path.join(d, "quotient_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", out, SRC, "-lm"], check=True)
    return out


@pytest.mark.parametrize("mode", ["bf16", "random"])
def test_quotient_is_ieee_division(exe, mode):
    args = [exe, mode] + (["20000000"] if mode == "random" else [])
    r = subprocess.run(args, capture_output=True, text=True, timeout=300)
    checked, bad = map(int, r.stdout.split())
    assert checked > 10_000_000 and bad == 0, (checked, bad)
