"""Build libdmu.so (HIP kernels for gfx950 + the C-ABI front end) in-tree.

    python -m dense_matrix_unit_amd.build

Every source is compiled with hipcc for gfx950 only.  Packed-FP32 instruction
selection is disabled for all device code.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdmu.so")
SOURCES = ["dmu_api.cpp", "gemm.hip", "gemm_block.hip", "gemm_skinny.hip", "quantize.hip",
           "probe.hip", "attention.hip"]
HEADERS = ["dmu_device.h", "dmu_internal.h", "gemm_common.h"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file code-generation options.  The block-scaled FP8 kernel promotes MFMA
# results with VALU FMAs, and the attention kernel rescales its output
# accumulators; VALU instructions cannot read AGPRs, so their MFMAs must write
# VGPRs.
EXTRA = {"gemm_block.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
