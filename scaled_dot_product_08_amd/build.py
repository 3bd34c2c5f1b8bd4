"""Build the gfx950 attention library in-tree with hipcc.

Produces ``scaled_dot_product_08_amd/lib/libsdpa08.so`` from the HIP kernel
and the C ABI layer. Run ``python -m scaled_dot_product_08_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libsdpa08.so")
SOURCES = ["attn_fwd_kernel.hip", "attn_fwd_fp8_kernel.hip", "attn_bwd_kernel.hip",
           "attn_decode_kernel.hip", "attn_clock.hip", "attn_api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU ops are switched off for all device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source to an object (in parallel) and link the shared library."""
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    base = [hipcc()] + HIPCC_FLAGS + list(extra_flags or []) + ["-I", os.path.join(ROOT, "include")]
    procs = []
    objs = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        cmd = base + ["-c", "-o", obj, os.path.join(CSRC, s)]
        cmd = [c for c in cmd if c != "-shared"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for s, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out + err)
            failed.append(s)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc link failed ({r.returncode})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
