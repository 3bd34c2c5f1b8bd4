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
           "attn_decode_kernel.hip", "attn_api.cpp"]
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


# Per-source extra flags. The forward file holds the one-wave-per-SIMD kernel
# (64 query rows per wave): with 512 registers available the compiler would
# otherwise give every MFMA accumulation-register operands, including the
# score blocks the softmax reads back at once. VGPR-form MFMAs leave the
# allocator free to keep the output accumulators and Q in the accumulation
# registers and the scores in VGPRs. (The other kernels of that file run two
# waves per SIMD and compile to identical code either way.)
SOURCE_FLAGS = {
    "attn_fwd_kernel.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                            "-Rpass-analysis=kernel-resource-usage"],
}
# Kernels that issue MFMAs from inline assembly: the compiler's hazard model
# does not cover those instructions, so any spill (scratch) or call inside
# them would put unguarded accesses next to in-flight MFMAs. The build fails
# if the resource report shows either.
ASM_MFMA_KERNELS = ("attn_fwd_w64_kernel",)


def check_asm_mfma_kernels(asm_path: str) -> None:
    """Fail unless every assembly-MFMA kernel in ``asm_path`` keeps its wait states."""
    try:
        from . import isa_check
    except ImportError:
        import isa_check
    with open(asm_path) as f:
        text = f.read()
    found = 0
    for part in ASM_MFMA_KERNELS:
        for name, body in isa_check.kernels(text, part).items():
            found += 1
            bad = isa_check.check(body)
            if bad:
                raise RuntimeError(f"{name}: {len(bad)} unguarded MFMA dependencies, e.g. {bad[0]}")
    if found == 0:
        raise RuntimeError("no assembly-MFMA kernel found in the forward assembly")


def check_resource_report(text: str) -> list[str]:
    """Kernels of ASM_MFMA_KERNELS whose resource report shows scratch or a dynamic stack."""
    bad = []
    name = None
    for line in text.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split()[0]
            continue
        if name is None or not any(k in name for k in ASM_MFMA_KERNELS):
            continue
        if "ScratchSize [bytes/lane]:" in line:
            if int(line.split("ScratchSize [bytes/lane]:")[1].split()[0]) != 0:
                bad.append(f"{name}: scratch")
        elif "Dynamic Stack:" in line and "True" in line.split("Dynamic Stack:")[1]:
            bad.append(f"{name}: dynamic stack")
    return bad


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
        cmd = base + SOURCE_FLAGS.get(s, []) + ["-c", "-o", obj, os.path.join(CSRC, s)]
        cmd = [c for c in cmd if c != "-shared"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    # The emitted assembly of the forward source, for the wait-state check of
    # its assembly MFMAs.
    asm_path = os.path.join(objdir, "attn_fwd_kernel.s")
    asm_cmd = [c for c in base if c != "-shared"] + SOURCE_FLAGS["attn_fwd_kernel.hip"] + \
        ["--cuda-device-only", "-S", "-o", asm_path, os.path.join(CSRC, "attn_fwd_kernel.hip")]
    asm_proc = subprocess.Popen(asm_cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    failed = []
    for s, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out + err)
            failed.append(s)
        elif "-Rpass-analysis=kernel-resource-usage" in SOURCE_FLAGS.get(s, []):
            bad = check_resource_report(out + err)
            if bad:
                raise RuntimeError(f"{s}: assembly-MFMA kernels must not spill or call: {bad}")
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    out, err = asm_proc.communicate()
    if asm_proc.returncode != 0:
        sys.stderr.write(out + err)
        raise RuntimeError("hipcc -S of the forward source failed")
    check_asm_mfma_kernels(asm_path)
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
