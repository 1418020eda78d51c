"""Builds liblogo.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m token_level_dynamic_amd.build

Every source is compiled with hipcc for gfx950 only, with packed fp32 VALU
instructions disabled, then linked into ``token_level_dynamic_amd/liblogo.so``.
Objects go to ``_build/`` at the repository root.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblogo.so")
# throughput-ceiling microbenchmarks for the benchmark's --ceilings mode: a
# library of their own, not linked into liblogo.so
CEILING_SRC = "ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libceiling.so")

SOURCES = ["abi.cpp", "select.hip", "attn_bf16.hip", "attn_f32.hip", "combine.hip",
           "backward_prep.hip", "backward_bf16.hip", "backward_f32.hip", "router.hip",
           "decode.hip"]
ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared libraries. Returns the path
    of the attention library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [CEILING_SRC]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
