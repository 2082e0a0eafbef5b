"""Build the HIP library libw4a16.so in-tree for gfx950 with hipcc.

Usage: python -m bf16_activation_quantized_amd.build   (or build() from Python)

Every translation unit is compiled with -O3 for gfx950 only; packed fp32
instructions are disabled for the device code (-packed-fp32-ops), and the
objects are linked into bf16_activation_quantized_amd/libw4a16.so.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4a16.so")

SOURCES = ["api.cpp", "pack_reduce.hip", "gemv.hip", "skinny.hip", "skinny_lds.hip", "prefill.hip"]
# MFMA accumulators that the VALU reads (diagonal extraction, per-group
# rescale) stay in VGPRs (the default heuristic moved them through AGPRs with
# extra copies); the decode GEMV's kernel arguments arrive preloaded in SGPRs
# (its first weight request waits on no scalar load)
EXTRA_FLAGS = {"gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=13"],
               "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "skinny_lds.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the W4A16 library)")


def _flags(src: str):
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
              "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
    if src.endswith(".hip"):
        common += ["-x", "hip", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    else:
        common += ["-x", "hip"]  # host-only code that includes hip_runtime.h
    common += EXTRA_FLAGS.get(src, [])
    return common


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
