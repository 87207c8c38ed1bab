"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host side (resolver, planner, C ABI, backward planning, and
the host parts of every kernel source: fits tests, tile choices, launch
wrappers) is compiled with both sanitizers on the host pass (the device
pass at -O0, only to give the objects their code objects), the oracle's C
loop nest likewise, all with ROCm's clang and its sanitizer runtimes, and
`sanitizer_driver.cpp` sweeps seeded descriptors --
valid ones and ones with one field broken -- through create, output shape,
workspace size, plan info and destroy for the forward, transposed and
backward handles, then runs the oracle on tiny problems with buffers
allocated at exactly their sizes.  No GPU call is made.  A sanitizer
finding aborts the driver; the test also fails on any report in its output.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

from convolution_implicit_gemm_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]
HOST_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", "-I", B.INCLUDE, "-I", B.CSRC]
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _sanitize_hipcc():
    # for hipcc, each sanitizer flag applies to the host pass only
    out = []
    for f in SAN:
        out += ["-Xarch_host", f]
    return out


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("hipcc") is None or not os.path.exists(CLANGXX):
        pytest.skip("hipcc / ROCm clang not available")
    out = str(tmp_path_factory.mktemp("asan"))
    jobs = [(s, None) for s in B.SOURCES] + [(s, k) for s in B.ACT_SOURCES for k in range(B.ACT_COUNT)]

    def compile_one(job):
        src, act = job
        stem = os.path.splitext(src)[0] + ("" if act is None else f"_a{act}")
        obj = os.path.join(out, stem + ".o")
        defs = [] if act is None else [f"-DFC_ACT={act}"]
        if src.endswith(".hip"):
            cmd = ["hipcc", f"--offload-arch={B.ARCH}", *HOST_FLAGS, "-Xarch_device", "-O0",
                   "-Xarch_device", "-g0", *_sanitize_hipcc(), *defs, "-x", "hip", "-c",
                   os.path.join(B.CSRC, src), "-o", obj]
        else:
            cmd = [CLANGXX, *HOST_FLAGS, *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                   *defs, "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, jobs))
    oracle_obj = os.path.join(out, "oracle.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c99", *SAN, "-fno-omit-frame-pointer", "-c",
                        os.path.join(ROOT, "oracle", "fusedconv_oracle.c"), "-o", oracle_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(out, "sanitizer_driver")
    r = subprocess.run([CLANGXX, *HOST_FLAGS, *SAN, os.path.join(ROOT, "tests", "sanitizer_driver.cpp"),
                        *objs, oracle_obj, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_host_code_under_asan_and_ubsan(driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "1"
    r = subprocess.run([driver, "3000"], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith(("library:", "oracle:"))]
    assert len(lines) == 2, r.stdout
    created = int(lines[0].split()[1])
    assert created > 300, lines[0]   # the sweep reaches the planner on many valid problems
    assert int(lines[1].split()[1]) > 50, lines[1]
