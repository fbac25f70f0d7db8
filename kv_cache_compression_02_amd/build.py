"""Build libkvc.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Each source is compiled to its own object in parallel, then the objects are
linked into one shared library.

Usage: python -m kv_cache_compression_02_amd.build
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvc.so")
SOURCES = ["api.hip", "snapkv.hip", "h2o.hip", "sink.hip", "decode.hip", "measure.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 instructions are left to the compiler's scalar forms only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result", "-Werror=return-type",
        "-I", INCLUDE, "-I", CSRC,
    ]


def object_path(src):
    return os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")


def compile_command(src):
    return [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", object_path(src)]


def link_command(out):
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[object_path(s) for s in SOURCES], "-o", out]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")
    return res


def build(verbose=True):
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        for r in list(ex.map(lambda s: _run(compile_command(s), verbose), SOURCES)):
            if r.stderr.strip() and verbose:
                sys.stderr.write(r.stderr)
    tmp = LIB + ".tmp"
    _run(link_command(tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
