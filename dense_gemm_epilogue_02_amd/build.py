"""Ahead-of-time build of the gfx950 GEMM library (``libmi355_gemm.so``).

Each HIP translation unit is compiled by ``hipcc --offload-arch=gfx950`` into
an object (in parallel), then linked into one shared library next to this
file. Packed fp32 VALU ops are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libmi355_gemm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["gemm_api.cpp", "kernels_generic.hip", "kernels_wholek.hip", "kernels_f32.hip",
           "kernels_f16.hip", "kernels_bf16.hip", "kernels_f8.hip", "kernels_mxf8.hip",
           "kernels_mxf4.hip"]

ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the GEMM library)")


def common_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + \
        common_flags() + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 0, extra=(), verbose: bool = False, only=None) -> str:
    """Compile every HIP source for gfx950 and link the shared library.
    ``only`` (a list of source names) recompiles just those and links the
    others' existing objects."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    todo = list(SOURCES) if only is None else [s for s in SOURCES if s in only]
    objs = {s: os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES
            if s not in todo}
    for s, o in objs.items():
        if not os.path.exists(o):
            raise RuntimeError(f"no object for {s}: build it first")
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, s, extra): s for s in todo}
        for f in cf.as_completed(futs):
            objs[futs[f]] = f.result()
            if verbose:
                print(f"compiled {futs[f]}", flush=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + \
        [objs[s] for s in SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    args = sys.argv[1:]
    only = [a for a in args if a in SOURCES] or None
    print(build(verbose=True, extra=[a for a in args if a not in SOURCES], only=only))
