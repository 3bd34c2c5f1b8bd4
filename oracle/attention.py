"""Plain float64 CPU attention forward: the oracle the GPU path is checked against.

TEST INFRASTRUCTURE. Nothing on the product path may import or call this
module; it shares no code with the HIP library.

What it computes (written from the pages, not from any listing):
  * Scaled dot-product attention per (batch, head):
    O = softmax(Q K^T * scale) V, the definition stated in
    mlqm.cn/news/343191 chapter 1 and its three-step unfused form
    (scores -> softmax over the key axis -> weighted sum of V) in the same
    chapter's PyTorch example and §2.1.
  * Causal masking: a score is kept when the key index does not exceed the
    query index and is replaced by -inf otherwise, as in the fused kernel of
    mlqm.cn/news/343191 §3.1 (its comparator was lost in extraction; the
    reading "key <= query is kept" is the only one consistent with a causal
    mask and with torch's ``is_causal``).
  * Packed variable-length batches: rows of one sequence attend only to keys
    of the same sequence, delimited by int32 prefix offsets ``cu_seqlens``
    (the varlen interface of lnrk.cn/news/11729 §1).
  * The per-row log-sum-exp of the scaled, masked logits, LSE = m + ln(l),
    where m is the row maximum and l the sum of exp(s - m): the two running
    statistics the online softmax of jianying88.com/news/49672 §3 keeps.
    The oracle does NOT use the online (tile by tile) form: it materialises
    the score rows and applies the plain definition, which the online form
    reaches exactly in exact arithmetic.

Arithmetic: float64 throughout. Inputs are the fp16/bf16 values the GPU
receives, upcast exactly. ``scale`` is used as given (callers pass the
float32 value the GPU receives).

  * Mask and bias variants (optional):
      - a sliding window of ``window`` keys with the first ``n_global``
        query rows of each sequence attending to every key: the
        window-plus-global-tokens scheme of lnrk.cn/news/11729 §2.5 (its
        listing computes full attention for the first 64 queries and
        sliding-window attention for the rest). Reading: row i >= n_global
        sees keys j with i - window < j <= i (causal) or |i - j| < window
        (non-causal); rows i < n_global see every key of the sequence.
      - ALiBi, the linear bias of jianying88.com/news/49672 §5.1 (named
        there, not written out). Reading: the standard per-head linear
        penalty, s_ij += -slope_h * |i - j|, added after scaling.

Parity pins (tests/test_oracle_*.py): pure-Python brute force on tiny
inputs, torch's CPU float64 scaled_dot_product_attention, and closed-form
invariants (rows sum to 1, equal scores give the mean of V and LSE = ln n,
causal row 0 returns V[0], permutation invariance, shift invariance,
argmax limit, packed == per-sequence; window >= length equals the plain
mask, zero slopes equal no bias).
"""
from __future__ import annotations

import numpy as np


def visible_mask(rows, L, causal, window=0, n_global=0):
    """Boolean (len(rows), L): which keys each query row may see (local indices)."""
    rows = np.asarray(rows)[:, None]
    keys = np.arange(L)[None, :]
    vis = np.ones((rows.shape[0], L), dtype=bool)
    if causal:
        vis &= keys <= rows
    if window > 0:
        if causal:
            vis &= keys > rows - window
        else:
            vis &= np.abs(keys - rows) < window
    if n_global > 0:
        vis |= rows < n_global
    return vis


def _head_rows(q, k, v, rows, causal, scale, window=0, n_global=0, slope=None):
    """Attention for the query ``rows`` (local indices) of one (sequence, head).

    q: (Lq_all, D) float64, k, v: (L, D) float64. Visible keys per
    ``visible_mask``; ``slope`` adds -slope * |i - j| to the scaled scores.
    Returns (O rows (n, Dv), LSE (n,), P (n, L) probabilities).
    """
    qi = q[rows]                                   # (n, D)
    s = (qi @ k.T) * scale                         # (n, L) logits, fp64
    L = k.shape[0]
    if slope is not None and slope != 0.0:
        dist = np.abs(np.asarray(rows)[:, None] - np.arange(L)[None, :])
        s = s - float(slope) * dist
    if causal or window > 0 or n_global > 0:
        s = np.where(visible_mask(rows, L, causal, window, n_global), s, -np.inf)
    m = s.max(axis=1)                              # row maximum
    w = np.exp(s - m[:, None])                     # exp(s - m); masked -> 0
    l = w.sum(axis=1)                              # row sum
    p = w / l[:, None]                             # softmax rows
    o = p @ v                                      # weighted sum of V
    lse = m + np.log(l)
    return o, lse, p


def attention(q, k, v, *, causal: bool, scale: float, cu_seqlens=None,
              return_probs: bool = False, window: int = 0, n_global: int = 0,
              alibi_slopes=None):
    """Full attention forward in float64.

    Padded mode (``cu_seqlens is None``): q, k, v are (B, S, H, D); returns
    O (B, S, H, D) and LSE (B, H, S).
    Packed mode: q, k, v are (T, H, D) and ``cu_seqlens`` is the int prefix
    offset array of length nseg+1; returns O (T, H, D) and LSE (H, T).
    With ``return_probs`` a dict {(seq, head): P} is returned as well
    (small inputs only). ``window``, ``n_global`` and ``alibi_slopes`` (one
    slope per head) select the mask and bias variants described above.
    """
    slopes = None if alibi_slopes is None else [float(x) for x in np.asarray(alibi_slopes)]
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    probs = {}
    if cu_seqlens is None:
        B, S, H, _ = q.shape
        o = np.zeros((B, S, H, v.shape[-1]))
        lse = np.zeros((B, H, S))
        rows = np.arange(S)
        for b in range(B):
            for h in range(H):
                ob, lb, pb = _head_rows(q[b, :, h], k[b, :, h], v[b, :, h], rows, causal, scale,
                                        window, n_global, None if slopes is None else slopes[h])
                o[b, :, h] = ob
                lse[b, h] = lb
                if return_probs:
                    probs[(b, h)] = pb
    else:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        T, H, _ = q.shape
        o = np.zeros((T, H, v.shape[-1]))
        lse = np.zeros((H, T))
        for s_idx in range(len(cu) - 1):
            a, e = cu[s_idx], cu[s_idx + 1]
            if e == a:
                continue
            rows = np.arange(e - a)
            for h in range(H):
                ob, lb, pb = _head_rows(q[a:e, h], k[a:e, h], v[a:e, h], rows, causal, scale,
                                        window, n_global, None if slopes is None else slopes[h])
                o[a:e, h] = ob
                lse[h, a:e] = lb
                if return_probs:
                    probs[(s_idx, h)] = pb
    if return_probs:
        return o, lse, probs
    return o, lse


def attention_rows(q, k, v, rows, *, causal: bool, scale: float, heads=None, window: int = 0,
                   n_global: int = 0, alibi_slopes=None):
    """Selected query rows of one padded-mode batch entry, all keys each row may see.

    q, k, v: (S, H, D) of a single batch entry (float64 or convertible);
    ``rows``: local query indices; ``heads``: head indices (default: all).
    Returns O (n_rows, n_heads, D) and LSE (n_heads, n_rows).
    Used at full sequence lengths, where materialising S x S is too large.
    """
    rows = np.asarray(rows, dtype=np.int64)
    H = q.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    o = np.zeros((len(rows), len(heads), v.shape[2]))
    lse = np.zeros((len(heads), len(rows)))
    kmax = int(rows.max()) + 1 if (causal and n_global == 0) else k.shape[0]
    slopes = None if alibi_slopes is None else [float(x) for x in np.asarray(alibi_slopes)]
    for hi, h in enumerate(heads):
        qh = np.asarray(q[:, h], dtype=np.float64)
        kh = np.asarray(k[:kmax, h], dtype=np.float64)
        vh = np.asarray(v[:kmax, h], dtype=np.float64)
        ob, lb, _ = _head_rows(qh, kh, vh, rows, causal, scale, window, n_global,
                               None if slopes is None else slopes[h])
        o[:, hi] = ob
        lse[hi] = lb
    return o, lse
