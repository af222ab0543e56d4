"""Build libmoe.so (the C-ABI library of include/moe.h) for gfx950 with hipcc.

Objects go to _build/ at the repository root; the shared library is written
next to this file so it travels with the package.  Every call recompiles (the
build is the "does it build" check); sources compile in parallel.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe.so")
# measurement support (model glue of the benchmark chain, ceiling kernels): a
# library of its own, never linked into libmoe.so
BENCH_SOURCES = ["bench_kernels.hip"]
BENCH_LIB = os.path.join(HERE, "libmoebench.so")
SOURCES = ["router.hip", "route.hip", "sort.hip", "gemv.hip", "decode.hip", "decode1.hip", "mfma.hip", "convert.hip", "api.cpp", "cache.cpp", "pipeline.cpp"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no hand-written or compiler-chosen packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results straight into VGPRs (no accumulation-register reads)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", "-pthread", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], BENCH_LIB)
    if verbose:
        print(f"built {LIB} and {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
