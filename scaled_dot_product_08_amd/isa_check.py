"""Wait-state check of MFMAs issued from inline assembly, on the compiler's gfx950 assembly.

The compiler inserts the wait states that MFMA dependencies need only for MFMAs it
generated itself. Instructions written as inline assembly (the accumulating MFMAs of
the 64-row-wave forward kernel, recognisable by their AGPR destination) are invisible
to it, so the build checks the emitted assembly of those kernels for the two
dependencies that the kernel guards by hand:

* a VALU instruction writes a VGPR that an assembly MFMA reads as A or B operand
  fewer than 2 wait states before it (gfx950 needs 2);
* any vector instruction reads or writes an accumulator (AGPR) that an assembly MFMA
  wrote fewer than 12 wait states before (gfx950 needs 12 after an 8-pass MFMA
  before a VALU read; memory instructions reading it, e.g. spills, need as many).

Wait states are counted as issued instructions, ``s_nop N`` counting N + 1; the
look-back ignores block labels (it follows the linear order, which covers the
fall-through path; a taken branch only adds instructions).
"""
from __future__ import annotations

import re

VALU_TO_MFMA = 2
MFMA_TO_ACC_ACCESS = 12


def _regs(tok: str) -> set:
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _instructions(text: str):
    out = []
    for n, raw in enumerate(text.splitlines()):
        line = raw.strip()
        if not line or line.startswith(";") or line.startswith("."):
            continue
        if line.endswith(":"):
            continue
        line = line.split(";")[0].strip()
        parts = line.replace(",", " ").split()
        out.append((parts[0], parts[1:], n + 1))
    return out


def _wait_states(op: str, args) -> int:
    return int(args[0], 0) + 1 if op == "s_nop" else 1


def _is_asm_mfma(op: str, args) -> bool:
    return op.startswith("v_mfma") and bool(args) and args[0].startswith("a[")


def check(text: str) -> list[str]:
    """Violations in one kernel's (or a whole file's) assembly text."""
    ins = _instructions(text)
    bad = []
    for k, (op, args, ln) in enumerate(ins):
        if _is_asm_mfma(op, args):
            srcs = _regs(args[1]) | _regs(args[2])
            w, j = 0, k - 1
            while j >= 0 and w < VALU_TO_MFMA:
                o2, a2, l2 = ins[j]
                if o2.startswith("v_") and not o2.startswith("v_mfma") and a2 and _regs(a2[0]) & srcs:
                    bad.append(f"line {l2} ({o2}) writes an operand of the MFMA at line {ln} "
                               f"{w} wait states before it")
                w += _wait_states(o2, a2)
                j -= 1
        if op.startswith(("v_", "scratch_", "buffer_", "global_", "ds_", "flat_")) and not op.startswith("v_mfma"):
            touched = set()
            for a in args:
                touched |= {r for r in _regs(a) if r[0] == "a"}
            if not touched:
                continue
            w, j = 0, k - 1
            while j >= 0 and w < MFMA_TO_ACC_ACCESS:
                o2, a2, l2 = ins[j]
                if _is_asm_mfma(o2, a2) and _regs(a2[0]) & touched:
                    bad.append(f"line {ln} ({op}) accesses an accumulator of the MFMA at line {l2} "
                               f"{w} wait states after it")
                w += _wait_states(o2, a2)
                j -= 1
    return bad


def kernels(text: str, name_part: str) -> dict:
    """Assembly of every kernel whose symbol contains ``name_part`` (label to s_endpgm)."""
    lines = text.splitlines()
    out = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S+):", l)
        if m and name_part in m.group(1):
            j = i
            while j < len(lines) and not lines[j].strip().startswith("s_endpgm"):
                j += 1
            out[m.group(1)] = "\n".join(lines[i:j + 1])
    return out
