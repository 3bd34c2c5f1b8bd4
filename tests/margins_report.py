"""Render the parity margins that the GPU tests record (ATTN_PARITY_REPORT=<json>) as the
markdown summary kept under profiles/.

    python tests/margins_report.py <margins.json> <out.md> [--tests N] [--source HASH]

Reads only the JSON the test session wrote; runs nothing on the GPU.
"""
from __future__ import annotations

import argparse
import json
import re
from collections import OrderedDict

WORKLOADS = ("tiny ", "mha ", "mha_causal ", "llama ", "long ", "varlen ")


def fmt(x) -> str:
    return "—" if x is None else f"{x:.2e}"


def group_of(case: str) -> str:
    """Mask-variant cases grouped by the shape they run on (dtype, D, padded or packed)."""
    m = re.match(r"mask variant B=(\d+) H=(\d+) S=(\d+) D=(\d+) (\w+) causal=", case)
    if m:
        return f"mask variants, padded B={m[1]} H={m[2]} S={m[3]} D={m[4]} {m[5]}"
    m = re.match(r"mask variant packed H=(\d+) D=(\d+) (\w+) causal=", case)
    if m:
        return f"mask variants, packed H={m[1]} D={m[2]} {m[3]} (lengths 1, 3, 0, 130, 257, 64, 200, 513)"
    return case


def render(d: dict, n_tests: int | None, source: str | None) -> str:
    cases = d["cases"]
    status = "all GPU tests passed" if d.get("exitstatus") == 0 else f"exit status {d.get('exitstatus')}"
    if n_tests:
        status += f" ({n_tests} tests)"
    out = ["# Parity margins of the five workloads and the mask variants (GPU vs the fp64 CPU oracle)",
           "",
           "Largest errors of the HIP library's output against the float64 oracle on the same seeded",
           "inputs, as recorded by the GPU parity tests, with the rounding floor of each case:",
           "max |RNE(O_ref) - O_ref|, the error that storing the exact output in the 16-bit type",
           "already makes (a lower bound for any kernel). Tolerances: O 4e-3 (fp16) / 1e-2 (bf16),",
           "LSE 1e-3. The mask variants are held to the O tolerance plus 2^-p |O_ref| per element",
           "(p = 8 significant bits for bf16, 11 for fp16; a narrow window or a steep slope makes",
           "|O| approach |V|), and to the same LSE tolerance.",
           "",
           "Command (on one MI355X, from the repository root, after building):",
           "",
           "```",
           "ATTN_PARITY_REPORT=/tmp/parity_margins.json python -u -m pytest tests -m gpu -x -q \\",
           "    --timeout 300 --timeout-method thread",
           "python tests/margins_report.py /tmp/parity_margins.json profiles/parity_margins.md",
           "```",
           "",
           f"Result: {status}" + (f"; forward kernel source `{source}`." if source else "."),
           "",
           "## The five workloads",
           "",
           "| workload (rows compared) | max\\|ΔO\\| | tol O | floor | ΔO / floor | max\\|ΔLSE\\| | tol LSE |",
           "|---|---|---|---|---|---|---|"]
    for c in cases:
        if not c["case"].startswith(WORKLOADS):
            continue
        ratio = (c["max_abs_dO"] / c["rne_floor_O"]) if c.get("rne_floor_O") else None
        out.append(f"| {c['case']} — {c['rows_checked']} rows | {fmt(c['max_abs_dO'])} | {c['tol_O']:g} | "
                   f"{fmt(c.get('rne_floor_O'))} | {'—' if ratio is None else f'{ratio:.2f}'} | "
                   f"{fmt(c['max_abs_dLSE'])} | {c['tol_LSE']:g} |")
    groups: "OrderedDict[str, list]" = OrderedDict()
    for c in cases:
        if c["case"].startswith("mask variant"):
            groups.setdefault(group_of(c["case"]), []).append(c)
    if groups:
        out += ["",
                "## Mask variants (sliding window, global rows, ALiBi), worst case of each group",
                "",
                "| group | cases | rows | max\\|ΔO\\| | its floor | worst case | worst ΔO − bound | max\\|ΔLSE\\| |",
                "|---|---|---|---|---|---|---|---|"]
        for g, cs in groups.items():
            w = max(cs, key=lambda c: c["max_abs_dO"])
            rows = sum(c["rows_checked"] or 0 for c in cs)
            tail = w["case"].split(" causal", 1)[1] if " causal" in w["case"] else w["case"]
            ex = [c["worst_excess_over_bound"] for c in cs if "worst_excess_over_bound" in c]
            out.append(f"| {g} | {len(cs)} | {rows} | {fmt(w['max_abs_dO'])} | {fmt(w.get('rne_floor_O'))} | "
                       f"causal{tail} | {fmt(max(ex)) if ex else '—'} | "
                       f"{fmt(max(c['max_abs_dLSE'] for c in cs))} |")
    ab = [c for c in cases if c["case"].startswith("alibi ")]
    if ab:
        out += ["",
                "## ALiBi alone on the 8-wave ping-pong kernel (same bound as the mask variants)",
                "",
                "| case | rows | max\\|ΔO\\| | floor | ΔO − bound | max\\|ΔLSE\\| |",
                "|---|---|---|---|---|---|"]
        for c in ab:
            out.append(f"| {c['case']} | {c['rows_checked']} | {fmt(c['max_abs_dO'])} | "
                       f"{fmt(c.get('rne_floor_O'))} | {fmt(c.get('worst_excess_over_bound'))} | "
                       f"{fmt(c['max_abs_dLSE'])} |")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("json_in")
    ap.add_argument("md_out")
    ap.add_argument("--tests", type=int, default=None, help="number of GPU tests the session ran")
    ap.add_argument("--source", default=None, help="forward kernel source hash the session ran")
    a = ap.parse_args()
    with open(a.json_in) as f:
        d = json.load(f)
    with open(a.md_out, "w") as f:
        f.write(render(d, a.tests, a.source))


if __name__ == "__main__":
    main()
