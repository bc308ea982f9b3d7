"""Builds ``libfa.so`` (the C-ABI attention library) for gfx950 with hipcc.

Usage: ``python -m tiled_attention_14_amd.build`` (or ``build()`` from Python).
Objects go to ``tiled_attention_14_amd/_build/``; the shared library is written
next to this file so it travels with the source tree.

Every compiler warning fails the build (the host pass's note that it does not
know the device-only ``packed-fp32-ops`` feature is the one line filtered
out).  The library embeds ``source_hash()`` of the sources and flags it was
built from; ``fa.lib()`` refuses a library whose hash differs from the tree's.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
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

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_splitkv.hip", "fa_fwd_fp8.hip", "fa_noalloc.hip"]

# Packed-fp32 VALU forms are disabled on purpose: only scalar fp32 VALU code is
# generated.  Float atomics are lowered to the hardware instructions.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def source_hash() -> str:
    """sha256 (16 hex digits) of every library source, the public header and the
    compile flags: what the built library must match."""
    h = hashlib.sha256()
    h.update(" ".join(HIP_FLAGS).encode())
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "fa.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


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
    if "warning" in out:
        raise RuntimeError(f"compiler warnings (the build treats them as errors): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    tag = source_hash()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        extra = ["-x", "hip"] if src.endswith(".hip") else [f'-DFA_SOURCE_HASH="{tag}"']
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
