"""Algorithmic work of one attention-forward call (the benchmark's metric).

FLOPs: two contractions per (batch, head), Q K^T and P V, each
2 * S * S * D multiply-adds counted as 2 FLOPs, i.e. 4 * S^2 * D per head
(jianying88.com/news/49672 §2 works this count for S=2048, D=64; the
per-operation form 2*b*h*n^2*d_k for Q K^T is in mlqm.cn/news/343191 §2.1).
Causal masking halves it (S^2/2 pairs, not S(S+1)/2: the metric's
convention). Packed sequences sum the per-sequence counts.

Bytes: the minimum HBM traffic of the fused method: Q, K, V read once,
O written once (2 bytes per element for fp16/bf16), LSE written once
(4 bytes per row per head). The pages count only Q/K/V reads (same §2).
"""
from __future__ import annotations

ELEM_BYTES = {"fp16": 2, "bf16": 2}


def flops(B: int, H: int, S: int, D: int, causal: bool) -> float:
    f = 4.0 * B * H * S * S * D
    return f / 2 if causal else f


def varlen_flops(lengths, H: int, D: int, causal: bool) -> float:
    return sum(flops(1, H, int(L), D, causal) for L in lengths)


def visible_pairs(L: int, causal: bool, window: int = 0, n_global: int = 0) -> int:
    """(query, key) pairs of one length-L sequence that the mask lets through.

    Rows below ``n_global`` see all L keys; any other row i sees keys j with
    j <= i (causal) and i - window < j (window > 0), or |i - j| < window
    when not causal.
    """
    import numpy as np
    g = min(max(n_global, 0), L)
    i = np.arange(g, L, dtype=np.int64)
    if causal:
        n = i + 1 if window <= 0 else np.minimum(i + 1, window)
    elif window <= 0:
        n = np.full(i.shape, L, dtype=np.int64)
    else:
        n = np.minimum(L - 1, i + window - 1) - np.maximum(0, i - window + 1) + 1
    return int(g) * int(L) + int(n.sum())


def masked_flops(B: int, H: int, L: int, D: int, causal: bool, window: int = 0,
                 n_global: int = 0) -> float:
    """4 * D FLOPs per visible pair (one D-long dot product, one D-long P V update).

    Used for the window / global-row variants, where the visible count is
    far from S^2/2 and the count itself is the meaningful work.
    """
    return 4.0 * D * B * H * visible_pairs(L, causal, window, n_global)


# The backward's algorithmic work: five products of the forward's size (the
# recomputed Q K^T, dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q) against
# the forward's two, i.e. 2.5x the forward count.
BACKWARD_FLOP_RATIO = 2.5


def qkv_read_bytes(B: int, H: int, S: int, D: int, dtype: str = "fp16") -> int:
    return 3 * B * H * S * D * ELEM_BYTES[dtype]


def min_hbm_bytes(B: int, H: int, S: int, D: int, dtype: str, with_lse: bool = True) -> int:
    """Q, K, V read once + O written once (+ fp32 LSE written once)."""
    e = ELEM_BYTES[dtype]
    n = 4 * B * H * S * D * e
    if with_lse:
        n += 4 * B * H * S
    return n


def logits_bytes(S: int, elem: int = 2) -> int:
    """Bytes of one (S x S) score matrix, what the fused method never stores."""
    return S * S * elem


def arithmetic_intensity(fl: float, nbytes: float) -> float:
    return fl / nbytes


def decode_bytes(B: int, H: int, Sq: int, D: int, lengths, dtype: str,
                 with_lse: bool = True) -> int:
    """Minimum HBM traffic of one decode step: the valid K and V cache rows
    read once, Q read once, O written once (+ fp32 LSE written once)."""
    e = ELEM_BYTES[dtype]
    rows = sum(int(L) for L in lengths)
    n = 2 * rows * H * D * e + 2 * B * Sq * H * D * e
    if with_lse:
        n += 4 * B * H * Sq
    return n


def decode_flops(H: int, Sq: int, D: int, lengths) -> float:
    """4 * D FLOPs per (query row, cache row) pair (non-causal count)."""
    return 4.0 * D * H * Sq * sum(int(L) for L in lengths)

