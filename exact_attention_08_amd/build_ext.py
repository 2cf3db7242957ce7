"""Build libfa355.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instructions
disabled, then linked into ``exact_attention_08_amd/libfa355.so``.  The same
sources built with -DFA_DEBUG_SYNC make the checking library
``libfa355_debug.so`` (every copy-pipeline wait drains all copies, LDS is
filled with NaN before first use); a GPU test requires its results to equal
the pipelined library's bit for bit.
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
DEBUG_LIB = os.path.join(PKG, "libfa355_debug.so")

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


def _compile(job) -> str:
    src, debug = job
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *(["-DFA_DEBUG_SYNC"] if debug else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}{' (debug)' if debug else ''}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in SOURCES]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
