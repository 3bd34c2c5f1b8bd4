"""Plain float64 CPU reference for attention against a KV cache (decode).

TEST INFRASTRUCTURE. Nothing on the product path may import or call this
module; it shares no code with the HIP library.

What it computes (written from the pages, not from any listing):
  * A few new query rows per sequence attend to the keys and values held in
    a KV cache laid out [batch, heads, seq_len, head_dim], the cache layout
    of lnrk.cn/news/11729 §2.2, which also notes that the cache grows by one
    row per generated token. The attention itself is the definition of
    mlqm.cn/news/343191 chapter 1: O = softmax(q K^T * scale) V per
    (sequence, head), with LSE = m + ln(l) as in jianying88.com/news/49672 §3.
  * Readings where the pages leave the decode step open:
      - ``seqlens_k[b]`` keys of the cache are valid for sequence b (all
        S_max when not given); the rest of the cache is ignored.
      - The Sq new query rows are the last Sq positions of the sequence:
        query row i sits at position L_b - Sq + i. Without causality every
        row sees all L_b valid keys; with causality row i sees keys
        j <= L_b - Sq + i (the mask of the full forward, aligned to the end).
      - A row that sees no key (L_b == 0, or L_b < Sq under causality) has
        O = 0 and LSE = -inf.
Arithmetic: float64 throughout; inputs are the fp16/bf16 values the GPU
receives, upcast exactly.

Parity pins (tests/test_oracle_decode.py): pure-Python brute force on tiny
inputs, torch's CPU float64 scaled_dot_product_attention with the explicit
end-aligned mask, and the reduction to the full forward (Sq = L_b with
causality is the causal forward of the first L_b tokens).
"""
from __future__ import annotations

import numpy as np


def decode_attention(q, k_cache, v_cache, *, causal: bool, scale: float, seqlens_k=None):
    """q (B, Sq, H, D); k_cache, v_cache (B, H, S_max, D).

    Returns O (B, Sq, H, Dv) and LSE (B, H, Sq), float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, Sq, H, _ = q.shape
    S_max = k_cache.shape[2]
    lens = [S_max] * B if seqlens_k is None else [int(x) for x in np.asarray(seqlens_k)]
    o = np.zeros((B, Sq, H, v_cache.shape[-1]))
    lse = np.full((B, H, Sq), -np.inf)
    for b in range(B):
        L = lens[b]
        for h in range(H):
            K = k_cache[b, h, :L]                      # valid keys (L, D)
            V = v_cache[b, h, :L]
            for i in range(Sq):
                n = L if not causal else min(L, max(0, L - Sq + i + 1))
                if n == 0:
                    continue                           # no visible key: O = 0, LSE = -inf
                s = (K[:n] @ q[b, i, h]) * scale       # logits of the visible keys
                m = s.max()
                w = np.exp(s - m)
                l = w.sum()
                o[b, i, h] = (w / l) @ V[:n]
                lse[b, h, i] = m + np.log(l)
    return o, lse
