"""Host-only build of the library's C++ host code under AddressSanitizer and UndefinedBehaviorSanitizer.

plan.cpp, block_plan.cpp, route.cpp and offload.cpp (descriptor checks, window and route tables,
plan and workspace layout, offload argument checks) are compiled for the host only with ROCm's
clang++, with csrc/host_stubs.cpp standing in for the kernel launchers, into
_build_san/libswinattn_san.so. tests/test_host_sanitizer.py runs the host tests against it
(SWIN_ATTN_LIB points the binding at it; the sanitizer runtime is preloaded). No GPU code is
built here. Usage: python shifted_window_attention_amd/build_host_sanitized.py
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build_san")
LIB = os.path.join(OUT_DIR, "libswinattn_san.so")
SOURCES = ["plan.cpp", "block_plan.cpp", "route.cpp", "offload.cpp", "host_stubs.cpp"]
CXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def runtime_libs():
    """The sanitizer runtimes to preload into the test process (clang's shared ASan runtime)."""
    out = subprocess.run([CXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return [out.stdout.strip()]


def build(verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [CXX, "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"] + SAN + \
              ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), r.stderr))
        objs.append(obj)
    cmd = [CXX, "-shared", "-shared-libsan"] + SAN + ["-o", LIB] + objs + ["-L/opt/rocm/lib", "-lamdhip64",
                                                                       "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
