"""Builds ``libfa.so`` (the C-ABI attention library) for gfx950 with hipcc.

Usage: ``python -m tiled_attention_14_amd.build`` (or ``build()`` from Python).
Objects go to ``tiled_attention_14_amd/_build/``; the shared library is written
next to this file so it travels with the source tree.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_splitkv.hip", "fa_fwd_fp8.hip"]

# Packed-fp32 VALU forms are disabled on purpose: only scalar fp32 VALU code is
# generated.  Float atomics are lowered to the hardware instructions.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfa.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        extra = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append((obj, [hipcc, *HIP_FLAGS, *inc, *extra, "-c", os.path.join(CSRC, src), "-o", obj]))
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[j[0] for j in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
