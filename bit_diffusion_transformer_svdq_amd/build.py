"""Builds libsvdq.so in-tree: HIP kernels for gfx950 plus the host-side C ABI and packer.

    python -m bit_diffusion_transformer_svdq_amd.build

Flags worth knowing:
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32 VALU
    instructions are emitted (the host pass prints a harmless warning about it);
  * ``-fhip-fp32-correctly-rounded-divide-sqrt`` and no fast-math: the kernels
    rely on IEEE division and fused multiply-add for bit-exact codes and scales;
  * the packer is compiled by g++ for x86-64-v3 (AVX2 + FMA).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libsvdq.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Wall", "-Wno-unused-function",
]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_API_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                  "-I", os.path.join(ROCM, "include")]
KERNELS = ["quant_lora_down.hip", "w4a4_gemm_lora_up.hip", "w4a4_gemm_skinny.hip", "fp4_gemm_big.hip",
           "awq_w4a16_gemm.hip"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required to build libsvdq")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    return res


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile every source and link libsvdq.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in KERNELS:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc, "-c", *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.insert(2, f"-save-temps={BUILD_DIR}")
            cmd[2] = "-save-temps=obj"
        _run(cmd, verbose)
        objs.append(obj)
    # the C ABI is host code: g++ against the HIP runtime API
    api_obj = os.path.join(BUILD_DIR, "api.o")
    _run(["g++", "-c", *HOST_API_FLAGS, "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, "api.cpp"),
          "-o", api_obj], verbose)
    objs.append(api_obj)
    packer_obj = os.path.join(BUILD_DIR, "packer.o")
    _run(["g++", "-c", "-O3", "-march=x86-64-v3", "-std=c++17", "-fPIC", "-Wall", "-fno-fast-math",
          "-ffp-contract=off", "-I", INCLUDE, os.path.join(CSRC, "packer.cpp"), "-o", packer_obj], verbose)
    objs.append(packer_obj)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp, "-lpthread"], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose=True, save_temps="--save-temps" in sys.argv)
    print(path)
