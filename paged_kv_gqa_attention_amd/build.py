"""Build libpa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m paged_kv_gqa_attention_amd.build

Compiles every source under csrc/ with hipcc for gfx950 and links
paged_kv_gqa_attention_amd/libpa.so.  Packed-FP32 VALU ops are disabled for the
device code (they are produced by the compiler only, never written by hand).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SOURCES = ["pa_kernels.hip", "pa_calib.hip", "pa_api.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, obj: str) -> None:
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = ["hipcc", "-x", "hip"] + DEVICE + COMMON + ["-c", path, "-o", obj]
    else:
        # host-only translation unit: HIP runtime API, no device code
        cmd = ["hipcc", "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")] + \
            COMMON + ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = True) -> str:
    """Compile all sources and link libpa.so; returns its path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda a: _compile(*a), zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
