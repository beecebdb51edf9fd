"""Build libmok.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m mixture_experts_layer_34_amd.build  (or build() from Python).
Objects go to _build/ at the repository root; the library lands next to this
file, so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmok.so")
DIAG = os.path.join(PKG, "libmok_diag.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["route_sort.hip", "permute_combine.hip", "gemm_bf16.hip", "gemm_stream.hip", "quantize_rows.hip", "gemm_f32.hip", "gemm_mxfp8.hip", "router_gemm.hip",
           "mok_abi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         # packed fp32 arithmetic stays off: hipcc would otherwise emit packed
         # fp32 add/mul/fma from plain float code.
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    # profiling driver (no PyTorch): runs the layer through the C ABI
    drv = os.path.join(PKG, "mok_profile")
    cmd = [HIPCC, *FLAGS, "-o", drv + ".tmp", os.path.join(CSRC, "mok_profile_main.cpp"), "-L" + PKG, "-lmok",
           "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("profiling driver build failed:\n" + r.stderr)
    os.replace(drv + ".tmp", drv)
    # matrix-core diagnostics (test support), a library of their own
    dobj = _compile("diag_mfma.hip")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", DIAG + ".tmp", dobj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("diagnostics link failed:\n" + r.stderr)
    os.replace(DIAG + ".tmp", DIAG)
    if verbose:
        print("built", OUT, "and", drv)
    return OUT


if __name__ == "__main__":
    build()
