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
