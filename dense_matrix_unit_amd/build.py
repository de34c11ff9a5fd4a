"""Build libdmu.so (HIP kernels for gfx950 + the C-ABI front end) in-tree.

    python -m dense_matrix_unit_amd.build

Every source is compiled with hipcc for gfx950 only.  Packed-FP32 instruction
selection is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
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


# a vector register operand, with or without modifiers (-v9, |v9|, -|v9|,
# neg(v9), sext(v9)): v9 or the range v[8:11]
_VREG = re.compile(r"(?<![\w.])v(?:\[(\d+):(\d+)\]|(\d+))(?!\w)")


def _vregs(text: str) -> set:
    """Every vector register named in `text` (an operand list)."""
    regs = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


def check_lds_asm_waits(src: str = "attention.hip") -> int:
    """The attention kernel issues its transposing LDS reads as inline
    assembly and waits on the LDS counter itself; the compiler does not know
    their registers fill later.  Scan the generated gfx950 code: between such
    a read and the s_waitcnt lgkmcnt that covers it (LDS reads complete in
    order), no instruction may read or write its destination.  Returns the
    number of reads checked; raises on a violation."""
    asm = os.path.join(BUILD, os.path.splitext(src)[0] + ".s")
    cmd = ([hipcc()] + COMMON + EXTRA.get(src, []) +
           ["-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", asm])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("assembly listing failed: %s\n%s" % (" ".join(cmd), r.stderr))
    with open(asm) as f:
        return scan_lds_asm_waits(f, asm)


def scan_lds_asm_waits(lines, name: str = "<listing>") -> int:
    """The check of check_lds_asm_waits over an assembly listing (an iterable
    of lines); returns the number of transposing reads checked.  While a read
    is pending (issued, its s_waitcnt lgkmcnt not yet reached), any
    instruction naming one of its destination registers in any operand --
    read, written, stored or used as an address, with or without modifiers --
    is an error, and so is a basic-block label or a branch: the scan follows
    the listing in order, so a pending read must not cross control flow."""
    pending, checked = {}, 0
    for n, line in enumerate(lines):
        t = line.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":"):
            if not t.startswith("."):
                pending = {}  # a new function
            elif pending:
                raise RuntimeError("%s:%d: label %s with hand-waited LDS reads pending"
                                   % (name, n + 1, t))
            continue
        if line[:1] not in (" ", "\t") or t[0] == ".":
            continue  # directives and other non-instruction lines
        op = t.split()[0]
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", t)
            if m:
                c = int(m.group(1))
                order = sorted(set(pending.values()))
                keep = set(order[len(order) - c:]) if c else set()
                pending = {reg: ln for reg, ln in pending.items() if ln in keep}
            continue
        if pending and op.startswith(("s_branch", "s_cbranch", "s_setpc", "s_swappc")):
            raise RuntimeError("%s:%d: branch with hand-waited LDS reads pending: %s"
                               % (name, n + 1, t))
        if op.startswith("s_"):
            continue
        operands = t[len(op):]
        if _vregs(operands) & set(pending):
            raise RuntimeError("%s:%d uses a transposing LDS read's registers before its "
                               "wait: %s" % (name, n + 1, t))
        if op == "ds_read_b64_tr_b16":
            checked += 1
            dest = operands.split(",")[0]
            for reg in _vregs(dest):
                pending[reg] = n
    if checked == 0:
        raise RuntimeError("%s: no transposing LDS reads found to check" % name)
    return checked


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
        checked = ex.submit(check_lds_asm_waits).result()
    if verbose:
        print("checked %d hand-waited LDS reads in the generated code" % checked)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
