"""The host C++ of the library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The two host-only sources (argument validation and planning in
minipic_api.cpp, the descriptor builder and block cache in descriptors.cpp)
are rebuilt with the sanitizers on their host code and linked with the
normally built kernels into a separate copy of the library; the CPU tests of
the boundary and of the descriptor builder then run against that copy in a
child process (the sanitizer runtime preloaded), and any report fails the
test. The pages' own engine shipped a double free in its block pool; this is
the check for that class of bug here.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "position_independent_paged_amd")
OUT = os.path.join(ROOT, "_build", "sanitize")
HOST_SOURCES = ["minipic_api.cpp", "descriptors.cpp"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _asan_runtime():
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return libs[0] if libs else None


@pytest.mark.slow
def test_host_code_under_sanitizers():
    cc, rt = _hipcc(), _asan_runtime()
    if cc is None or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not installed")
    sys.path.insert(0, PKG)
    import build as lib_build
    kernel_objs = []
    for src in lib_build.sources():
        obj = os.path.join(lib_build.BUILD, os.path.basename(src) + ".o")
        if os.path.basename(src) not in HOST_SOURCES:
            if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(src):
                pytest.skip("kernels not built: run position_independent_paged_amd/build.py first")
            kernel_objs.append(obj)
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for name in HOST_SOURCES:
        obj = os.path.join(OUT, name + ".o")
        flags = [f for f in lib_build.compile_flags(debug=True)]
        cmd = [cc] + flags + SAN + ["-c", os.path.join(PKG, "csrc", name), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    lib = os.path.join(OUT, "libminipic_sanitized.so")
    cmd = [cc, f"--offload-arch={lib_build.ARCH}", "-shared", "-fPIC", "-shared-libsan", "-o", lib] + objs + \
        kernel_objs + SAN
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, MINIPIC_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow",
                        "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_host_cpu.py"),
                        os.path.join(ROOT, "tests", "test_descriptors.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    text = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, text
    assert "ERROR: AddressSanitizer" not in text and "runtime error:" not in text, text
    assert "passed" in r.stdout
