"""Builds the HIP library ``liblh.so`` for gfx950 next to this file.

Usage: ``python -m nvfp4_scale_calibration_lh_amd.build`` (or ``build()`` from Python).  Every call
recompiles; objects go to ``_build/`` in the package directory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblh.so")
SOURCES = ["absmax.hip", "accumulate.hip", "sweep.hip", "dequant.hip", "lh_abi.cpp"]
ARCH = "gfx950"
# Packed fp32 ALU instructions are kept out of the generated code; MFMA results live in VGPRs
# (no accumulator-register copies in the sweep loop).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-Wall",
         "-Wno-unused-function"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stdout + p.stderr).splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([hipcc, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for msg in ex.map(_run, cmds):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = OUT + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
