import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU oracle runs")


def pytest_sessionstart(session):
    # build the HIP library once if it is missing (tests load what is built)
    import importlib.util
    lib = os.path.join(ROOT, "shifted_window_attention_amd", "libswinattn.so")
    if not os.path.exists(lib):
        spec = importlib.util.spec_from_file_location(
            "swin_build_lib", os.path.join(ROOT, "shifted_window_attention_amd", "build_lib.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(verbose=True)
