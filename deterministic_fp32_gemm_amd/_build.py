"""Ahead-of-time build of libsdm_gx_gemm.so for gfx950 with hipcc (in-tree, no JIT cache)."""

from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libsdm_gx_gemm.so")
SOURCES = ("gx_gemm_kernel.hip", "gx_gemm_mfma.hip", "gx_gemm_api.cpp", "gx_pa2_kernel.hip", "gx_pa2_api.cpp")

# Numerics-relevant flags: no contraction or fast-math (the chain's fmaf and the final add are what runs), f32
# denormals kept, and no packed-FP32 instructions (scalar v_fma_f32 / v_fmac_f32 only).
HIP_FLAGS = (
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall",
)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsdm_gx_gemm)")


def build(out: str = LIB_PATH, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library (always recompiles)."""
    objs = []
    tmpdir = os.path.join(PKG, "_objs")
    os.makedirs(tmpdir, exist_ok=True)
    cc = hipcc()
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
