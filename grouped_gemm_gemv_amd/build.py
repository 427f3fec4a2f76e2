"""Build libmoe.so (the layer), libmoe_peaks.so (measurement probes) and
libmoe_phases.so (the layer with main-loop phase timing in its bf16 grouped
GEMMs, for measurement only) in-tree with hipcc for gfx950.

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
PHASES_LIB = os.path.join(PKG, "libmoe_phases.so")
ARCH = "gfx950"
SOURCES = ["api.cpp", "route.hip", "dispatch.hip", "gemm_bf16_gateup.hip", "gemm_bf16_down.hip",
           "gemm_f32_gateup.hip", "gemm_f32_down.hip", "gemm_fp8w_gateup.hip", "gemm_fp8w_down.hip", "layout.hip",
           "noalloc.hip"]
PEAKS_SOURCES = ["peaks.hip"]
# recompiled with MOE_LOOP_PHASES for libmoe_phases.so (the other objects are shared)
PHASES_SOURCES = ["gemm_bf16_gateup.hip", "gemm_bf16_down.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(job) -> str:
    src, phases = job
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ("_phases.o" if phases else ".o"))
    cmd = [hipcc()] + common_flags() + (["-DMOE_LOOP_PHASES"] if phases else []) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
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
    jobs = [(s, False) for s in SOURCES + PEAKS_SOURCES] + [(s, True) for s in PHASES_SOURCES]
    with ThreadPoolExecutor(len(jobs)) as ex:
        objs = dict(zip(jobs, ex.map(_compile, jobs)))
    _link([objs[(s, False)] for s in SOURCES], LIB)
    _link([objs[(s, False)] for s in PEAKS_SOURCES], PEAKS_LIB)
    _link([objs[(s, s in PHASES_SOURCES)] for s in SOURCES], PHASES_LIB)
    if verbose:
        print(f"built {LIB}, {PEAKS_LIB} and {PHASES_LIB}")
    return LIB


if __name__ == "__main__":
    build()
