import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # tests load the built library; build it only if nothing is built yet
    lib = os.path.join(ROOT, "fp8_block_quantized_amd", "libmoe_fp8.so")
    if not os.path.exists(lib):
        from fp8_block_quantized_amd import build
        build.build()
