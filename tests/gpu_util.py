"""Helpers for the GPU tests: move seeded inputs to the device and compare with the oracle."""
import sys

import numpy as np
import torch

import synth

TOL_O = {"fp16": 4e-3, "bf16": 1e-2}   # max-abs on O
TOL_LSE = 1e-3                          # max-abs on LSE
TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def scale_of(D: int) -> float:
    return float(np.float32(1.0 / np.sqrt(D)))


def max_abs(a, b) -> float:
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    if np.isnan(d).any():
        return float("inf")
    return float(d.max()) if d.size else 0.0


# ---- parity margins ------------------------------------------------------------
# Tests that compare a workload with the oracle record their largest errors here;
# conftest.py writes them out at the end of the session when ATTN_PARITY_REPORT
# names a file.
MARGINS: list = []


def rne_floor(oref: np.ndarray, dtype: str) -> float:
    """max |RNE(oref) - oref|: the error that rounding the exact output to the storage
    type alone already makes (round to nearest even, computed from float64)."""
    x = np.asarray(oref, np.float64)
    if x.size == 0:
        return 0.0
    if dtype == "fp16":
        r = x.astype(np.float16).astype(np.float64)
    else:
        # bf16 keeps 8 significant bits: round to a multiple of 2^(e-7), ties to even
        # (numpy's round is half-to-even); zeros and subnormal-range values stay as is.
        ax = np.abs(x)
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
        ulp = np.exp2(e - 7)
        r = np.where(ax > 0, np.round(x / ulp) * ulp, x)
    return float(np.abs(r - x).max())


def record(case: str, dtype: str, eo: float, el: float, oref=None, n_rows: int | None = None,
           floor: float | None = None, tol_o: float | None = None, excess: float | None = None):
    """Remember one case's largest errors (and the rounding floor of its exact output).
    ``excess``: for cases held to a per-element bound, the largest |dO| minus that bound
    (at most 0 when the case passes)."""
    if floor is None and oref is not None:
        floor = rne_floor(oref, dtype)
    rec = {"case": case, "dtype": dtype, "max_abs_dO": eo, "max_abs_dLSE": el,
           "tol_O": TOL_O[dtype] if tol_o is None else tol_o, "tol_LSE": TOL_LSE,
           "rne_floor_O": floor, "rows_checked": n_rows}
    if excess is not None:
        rec["worst_excess_over_bound"] = excess
    MARGINS.append(rec)
