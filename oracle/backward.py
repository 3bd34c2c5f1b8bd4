"""Plain float64 CPU reference for the attention backward pass (dQ, dK, dV).

TEST INFRASTRUCTURE. Nothing on the product path may import or call this
module; it shares no code with the HIP library.

What it computes: the gradients of the forward of oracle/attention.py,
O = softmax(scale * Q K^T + mask) V per (sequence, head), with respect to
Q, K and V, given the gradient dO of a loss with respect to O. The pages
reserve a backward(grad_output) entry point and a gradient mask for the
fused operation (mlqm.cn/news/343191 §3.3) without writing it out; the
reading taken here is the chain rule through the three steps of the
forward (scores -> row softmax -> weighted sum of V), written for one
(sequence, head) with P the probabilities:
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))        (softmax Jacobian, row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q
Masked entries have P = 0 and therefore dS = 0. rowsum(P * dP) equals
rowsum(dO * O), the form the GPU path uses; here it is taken from P and dP.
Arithmetic: float64 throughout; inputs are the fp16/bf16 values the GPU
receives, upcast exactly.

Parity pins (tests/test_oracle_backward.py): central finite differences of
the forward oracle, torch's CPU float64 autograd through
scaled_dot_product_attention, and closed forms (dK sums to zero over the
keys of a (sequence, head); dV sums to the sum of dO; zero scale gives
dQ = dK = 0 and dV = column means of dO).
"""
from __future__ import annotations

import numpy as np

from .attention import visible_mask


def _head_backward(q, k, v, do, causal, scale):
    """One (sequence, head): q, do (L, D); k, v (L, D). Returns dq, dk, dv."""
    L = q.shape[0]
    s = (q @ k.T) * scale
    if causal:
        s = np.where(visible_mask(np.arange(L), L, True), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    p = w / w.sum(axis=1, keepdims=True)          # probabilities, masked -> 0
    dv = p.T @ do
    dp = do @ v.T
    delta = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - delta)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, dout, *, causal: bool, scale: float, cu_seqlens=None):
    """Gradients of the attention forward.

    Padded mode: q, k, v, dout (B, S, H, D); packed mode: (T, H, D) with
    ``cu_seqlens``. Returns dq, dk, dv in the layout of q, k, v (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if cu_seqlens is None:
        B, S, H, _ = q.shape
        for b in range(B):
            for h in range(H):
                g = _head_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], causal, scale)
                dq[b, :, h], dk[b, :, h], dv[b, :, h] = g
    else:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        H = q.shape[1]
        for i in range(len(cu) - 1):
            a, e = cu[i], cu[i + 1]
            if e == a:
                continue
            for h in range(H):
                g = _head_backward(q[a:e, h], k[a:e, h], v[a:e, h], do[a:e, h], causal, scale)
                dq[a:e, h], dk[a:e, h], dv[a:e, h] = g
    return dq, dk, dv
