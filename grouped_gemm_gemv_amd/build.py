"""Build libmoe.so (the layer) and libmoe_peaks.so (measurement probes)
in-tree with hipcc for gfx950.

    python -m grouped_gemm_gemv_amd.build

Every HIP source is compiled for gfx950 only.  Packed-fp32 instructions are
switched off for device code (the hipcc host pass warns that it does not know
the feature; that warning is harmless).
"""
from __future__ import annotations

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
LIB = os.path.join(PKG, "libmoe.so")
PEAKS_LIB = os.path.join(PKG, "libmoe_peaks.so")
ARCH = "gfx950"
SOURCES = ["api.cpp", "route.hip", "dispatch.hip", "gemm_bf16_gateup.hip", "gemm_bf16_down.hip",
           "gemm_f32_gateup.hip", "gemm_f32_down.hip", "gemm_fp8w_gateup.hip", "gemm_fp8w_down.hip", "layout.hip",
           "noalloc.hip"]
PEAKS_SOURCES = ["peaks.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build()
