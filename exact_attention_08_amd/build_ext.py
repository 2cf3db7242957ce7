"""Build libfa355.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instructions
disabled, then linked into ``exact_attention_08_amd/libfa355.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa355.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_wide.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fwd_fp8.hip"]
# MFMA results of the forward kernel are consumed by VALU code (the softmax):
# keep them in arch VGPRs instead of accumulation registers.  Its arithmetic
# never makes a NaN from finite inputs, so NaNs need not be honoured: v_max
# then takes MFMA results directly instead of after a quieting copy each.
EXTRA = {"fa_fwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
         "fa_fwd_wide.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
         "fa_bwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
