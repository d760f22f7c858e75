"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

plan.cpp, block_plan.cpp, route.cpp and offload.cpp are rebuilt for the host only with
-fsanitize=address,undefined (kernel launchers stubbed), and the host test files run against that
build in a child process with the sanitizer runtime preloaded. Any out-of-bounds access, use after
free or undefined behaviour in the descriptor checks, window tables, route planner or plan
layout aborts the child, and this test fails with its report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "shifted_window_attention_amd"))

HOST_TESTS = ["tests/test_abi_host.py", "tests/test_route_host.py", "tests/test_host_fuzz.py"]


def test_host_code_is_clean_under_asan_and_ubsan():
    import build_host_sanitized as B
    try:
        lib = B.build()
    except (OSError, RuntimeError) as e:  # no clang++ with sanitizer runtimes in this image
        pytest.skip("sanitized host build unavailable: %s" % e)
    rt = B.runtime_libs()
    if not all(os.path.exists(p) for p in rt):
        pytest.skip("sanitizer runtime not found: %s" % rt)
    env = dict(os.environ)
    env["SWIN_ATTN_LIB"] = lib
    env["LD_PRELOAD"] = ":".join(rt + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    # Leak checking is off: the Python interpreter and torch keep allocations alive to exit.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = ROOT + ((":" + env["PYTHONPATH"]) if env.get("PYTHONPATH") else "")
    # The child really runs the sanitized build with the runtime in the process.
    probe = ("import ctypes; from shifted_window_attention_amd import native; "
             "assert native.LIB_PATH == %r, native.LIB_PATH; ctypes.CDLL(None)['__asan_init']; "
             "ctypes.CDLL(native.LIB_PATH)['__ubsan_handle_add_overflow']; print('sanitized')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "sanitized" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"]
                       + HOST_TESTS, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
