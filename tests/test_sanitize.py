"""Sanitizer runs on the CPU: the C oracle and the library's host runtime
built with AddressSanitizer + UndefinedBehaviorSanitizer (errors fatal),
each driven over a grid of shapes, options and invalid arguments by a small
C program under tests/sanitize/.  No GPU: the host runtime's calls all end in
argument checks, plans and sizes (the device code is built, never run).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "sparse_selection_primitive_amd")
CLANG = "/opt/rocm/lib/llvm/bin/clang"
SAN_FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, env_extra=None, timeout=600):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    res = _run(["gcc", "-std=c11", "-fopenmp", *SAN_FLAGS, os.path.join(ROOT, "oracle", "lapsum_oracle.c"),
                os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    assert res.returncode == 0, res.stderr
    res = _run([exe], {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1", "OMP_NUM_THREADS": "4"})
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all checks passed" in res.stdout
    assert "runtime error" not in res.stderr


def _sanitized_library():
    """The host-sanitized build of the library, rebuilt when a source is newer."""
    from sparse_selection_primitive_amd import build
    out = os.path.join(PKG, "_build", "liblapsum_hostsan.so")
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)] + [os.path.join(ROOT, "include", "lapsum.h")]
    if not os.path.exists(out) or os.path.getmtime(out) < max(os.path.getmtime(s) for s in srcs):
        os.makedirs(os.path.dirname(out), exist_ok=True)
        build.build_host_sanitized(out)
    return out


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_host_runtime_under_asan_ubsan(tmp_path):
    lib = _sanitized_library()
    exe = str(tmp_path / "host_driver")
    res = _run([CLANG, *SAN_FLAGS, "-I", os.path.join(ROOT, "include"), os.path.join(SAN, "host_driver.c"), "-o",
                exe, lib, f"-Wl,-rpath,{os.path.dirname(lib)}", "-L/opt/rocm/lib", "-lamdhip64",
                "-Wl,-rpath,/opt/rocm/lib", "-lstdc++", "-lm"])
    assert res.returncode == 0, res.stderr
    # leak checking is off: the HIP runtime keeps allocations until exit
    res = _run([exe], {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"})
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all checks passed" in res.stdout
    assert "runtime error" not in res.stderr
