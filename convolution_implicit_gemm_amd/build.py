"""Build libfusedconv.so in-tree with hipcc for gfx950.

Usage: python -m convolution_implicit_gemm_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfusedconv.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["resolver.cpp", "planner.cpp", "capi.cpp", "kernels_direct.hip", "kernels_igemm.hip",
           "kernels_transposed.hip", "kernels_im2col.hip", "noalloc.hip", "backward.cpp",
           "kernels_backward.hip", "kernels_halo32.hip"]
# Kernels specialised per activation: compiled once per activation id
# (-DFC_ACT=k, k = 0 .. ACT_COUNT-1); unit 0 also holds the route entry points.
ACT_SOURCES = ["kernels_depthwise.hip", "kernels_dwmfma.hip", "kernels_halo.hip",
               "kernels_smallc.hip", "kernels_pointwise.hip"]
ACT_COUNT = 15
ARCH = "gfx950"
# Packed fp32 ops stay off (the compiler is not allowed to form v_pk_*_f32).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def _compile(job) -> str:
    src, act = job
    stem = os.path.splitext(src)[0] + ("" if act is None else f"_a{act}")
    obj = os.path.join(BUILD, stem + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    defs = [] if act is None else [f"-DFC_ACT={act}"]
    cmd = ["hipcc", *FLAGS, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {stem}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(f, k) for f in ACT_SOURCES for k in range(ACT_COUNT)] + [(f, None) for f in SOURCES]
    workers = max(1, min(16, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, jobs))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                           *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
