"""Build liblapsum.so (the C-ABI HIP library) in-tree for gfx950.

    python -m sparse_selection_primitive_amd.build

Every translation unit is compiled by hipcc for gfx950 only, with packed
fp32 instructions disabled, then linked into one shared library next to this
file.  Object files go to ``_build/`` (not tracked).

``build_lds_poison()`` builds a debug copy whose kernels fill their LDS with
0xFF bytes at entry (``liblapsum_ldspoison.so``, loaded only by its GPU test).

``build_host_sanitized(path)`` builds a second copy of the library for CPU
checks of the host runtime: its host code instrumented with AddressSanitizer
and UndefinedBehaviorSanitizer (the device code is built as usual, without
them).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblapsum.so")
SOURCES = ["api.cpp", "onchip.hip", "stream.hip", "bracket.hip", "band.hip", "sort.hip", "bisect.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _flags():
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str, objdir: str = BUILD, defines=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *_flags(), *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def build_host_sanitized(out: str, jobs: int | None = None) -> str:
    """Host-only ASan + UBSan build of every translation unit, linked to
    ``out``.  The sanitizer runtime is not linked in: the program that loads
    the library must carry it (a sanitized executable, or the runtime
    preloaded)."""
    objdir = out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    flags = ["-x", "hip", f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(HERE, "..", "include")]

    def one(src: str) -> str:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        res = subprocess.run([hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj], capture_output=True,
                             text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitized host build failed for {src}:\n{res.stderr}")
        return obj

    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    res = subprocess.run([hipcc(), "-shared", "-fPIC", "-o", out, *objs], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized host link failed:\n{res.stderr}")
    return out


def build(jobs: int | None = None, out: str = LIB, defines=()) -> str:
    objdir = BUILD if not defines else os.path.join(BUILD, "_".join(d.lower() for d in defines))
    os.makedirs(objdir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, objdir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    return out


POISON_LIB = os.path.join(HERE, "liblapsum_ldspoison.so")


def build_lds_poison(jobs: int | None = None) -> str:
    """The debug copy of the library whose kernels set their LDS to 0xFF
    bytes at entry (LAPSUM_LDS_POISON), for the GPU test that runs the
    parity cases against it."""
    return build(jobs, POISON_LIB, ("LAPSUM_LDS_POISON",))


if __name__ == "__main__":
    print(build())
