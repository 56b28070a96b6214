"""Builds libmuon.so (HIP kernels + C ABI) in-tree for gfx950.

    python -m newton_schulz_10_amd.build        # or build_library()

Each source compiles to an object under newton_schulz_10_amd/_build/, then
everything links into newton_schulz_10_amd/libmuon.so. hipcc cross-compiles
for gfx950 without a GPU present.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmuon.so")

SOURCES = ["plan.cpp", "muon_api.cpp", "elementwise.hip", "gemm_bf16.hip", "gemm_f32.hip", "scratch.hip"]
ARCH = os.environ.get("MUON_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            f"--offload-arch={ARCH}",
            # Packed fp32 VALU forms are kept out of the generated code.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # Atomics stay single instructions: the GEMM's tile claim (one
            # lane) must not be rewritten into a wave reduction that uses
            # its result, and so waits for it, right away.
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc()] + common_flags() + ["-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + \
          ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-soname,libmuon.so", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libmuon.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
