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
