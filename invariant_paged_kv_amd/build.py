"""Compile the HIP library ``libbia.so`` in-tree for gfx950.

``python -m invariant_paged_kv_amd.build`` (or ``build_library()``) runs hipcc
on ``csrc/plan.cpp`` and ``csrc/bia.hip``. Packed-fp32 instruction selection
is turned off (``-packed-fp32-ops``); hipcc's host pass warns that it does not
know the feature, which is harmless. MFMAs are selected in their VGPR form
(``-amdgpu-mfma-vgpr-form``): the latent kernels, which run one wave per SIMD
with more than 256 registers, otherwise copy their output accumulators
between the VGPR and AGPR files on every tile; no other kernel's code changes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libbia.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = os.environ.get("BIA_OFFLOAD_ARCH", "gfx950")

SOURCES = [os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "bia.hip")]
HEADERS = [os.path.join(INCLUDE, "bia.h"), os.path.join(CSRC, "plan.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_command(out: str = LIB_PATH) -> list:
    return [
        hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-shared", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *SOURCES, "-o", out,
    ]


def build_library(verbose: bool = False) -> str:
    """Always recompiles; writes to a temporary name and renames atomically."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
