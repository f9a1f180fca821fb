"""Sanitizer leg of the CPU suite: AddressSanitizer + UndefinedBehaviorSanitizer
builds of the host code, exercised by the CPU tests.

Two libraries are rebuilt with -fsanitize=address,undefined (UB made fatal):
the fp64 oracle (oracle/pa_oracle.c, gcc) and the host layer of libpa.so
(pa_api.cpp: planning, argument validation, workspace layout, the static
scratch entry point's checks), compiled with g++ and linked with the normal
gfx950 device object.  A child Python process with the ASan runtime preloaded
points the binding and the oracle at them and runs the CPU tests (without
the GPU, the runs stop at validation: nothing is launched).  Any sanitizer
report fails the child and this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_gqa_attention_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
from paged_kv_gqa_attention_amd import binding as B
B.LIB_PATH = {lib!r}
import oracle
oracle._lib = oracle.load({olib!r})
import pytest
sys.exit(pytest.main([{tests!r}, "-m", "not gpu", "-q", "-x", "-p", "no:cacheprovider",
                      "--deselect", {mut!r}, "--deselect", {me!r}]))
"""


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    if os.environ.get("PA_SANITIZED_CHILD"):
        pytest.skip("already inside the sanitized run")
    # the device-code objects of libpa.so as build.py compiled them
    kobjs = [os.path.join(PKG, "_build", s + ".o") for s in ("pa_kernels.hip", "pa_calib.hip")]
    if not all(os.path.exists(k) for k in kobjs):
        pytest.skip("libpa.so has not been built (python -m paged_kv_gqa_attention_amd.build)")
    olib = str(tmp_path / "libpa_oracle_san.so")
    run(["gcc", "-O1", "-std=c99", "-fopenmp", "-shared", "-fPIC"] + SAN +
        ["-I", os.path.join(ROOT, "oracle"), "-o", olib, os.path.join(ROOT, "oracle", "pa_oracle.c"), "-lm"])
    aobj = str(tmp_path / "pa_api_san.o")
    run(["g++", "-O1", "-std=c++17", "-fPIC"] + SAN +
        ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(PKG, "csrc"), "-c", os.path.join(PKG, "csrc", "pa_api.cpp"), "-o", aobj])
    lib = str(tmp_path / "libpa_san.so")
    run(["g++", "-shared"] + SAN + ["-o", lib, aobj] + kobjs + ["-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                                    "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    asan = run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, PA_SANITIZED_CHILD="1", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # node ids relative to the repository root (the child's working directory)
    code = CHILD.format(root=ROOT, lib=lib, olib=olib, tests="tests",
                        mut="tests/test_oracle_mutants.py", me="tests/test_sanitizers.py")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=900)
    log = r.stdout[-6000:] + r.stderr[-6000:]
    assert "ERROR: AddressSanitizer" not in log and "runtime error:" not in log, log
    assert r.returncode == 0, log
    assert " passed" in r.stdout, log
