"""Float64 CPU reference for attention on FP8 (E4M3) inputs with per-tensor scales.

TEST INFRASTRUCTURE. Nothing on the product path may import or call this
module; it shares no code with the HIP library.

What it computes: jianying88.com/news/49672 §3 mentions FP8 for the fused
attention (FlashAttention-2's FP8 mode: little TFLOPS gain, less memory) and
gives no format. The reading taken here: Q, K and V are stored as 8-bit
floats in the OCP E4M3 format (1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; the single
pattern S.1111.111 is NaN; no infinities; largest finite value 448), each
tensor with one float scale ("descale") that multiplies every decoded value.
The attention is then the plain definition of oracle/attention.py applied to
descale_q * Q, descale_k * K and descale_v * V, in float64.

Parity pins (tests/test_oracle_fp8.py): the decoder against torch's
float8_e4m3fn for all 256 codes, the encoder against the same on random and
boundary values (round to nearest even, overflow to NaN), and the reduction
of the attention to oracle.attention on the decoded inputs.
"""
from __future__ import annotations

import numpy as np

from .attention import attention


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 bit patterns (uint8) -> float64, from the format's definition."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """float -> OCP E4M3 bit patterns, round to nearest even; |x| above 464
    (halfway from 448 to the next step, which would be the NaN pattern; the
    tie itself goes to the even 448) and NaN give 0x7F (sign kept)."""
    x = np.asarray(x, dtype=np.float64)
    table = e4m3_decode(np.arange(128))            # non-negative codes 0..127
    finite = np.arange(127)                        # 0x7F is NaN
    vals = table[finite]
    out = np.zeros(x.shape, dtype=np.int64)
    ax = np.abs(x)
    for idx in np.ndindex(x.shape):
        a = ax[idx]
        if np.isnan(a) or a > 464.0:
            out[idx] = 0x7F
        else:
            j = int(np.searchsorted(vals, a))      # vals[j-1] < a <= vals[j]
            if j == 0:
                out[idx] = 0
            else:
                lo, hi = vals[j - 1], vals[min(j, 126)]
                if j > 126 or a - lo < hi - a:
                    out[idx] = j - 1
                elif a - lo > hi - a:
                    out[idx] = j
                else:                              # tie: even mantissa (even code)
                    out[idx] = j - 1 if (j - 1) % 2 == 0 else j
        if np.signbit(x[idx]):
            out[idx] |= 0x80
    return out.astype(np.uint8)


def attention_fp8(q8, k8, v8, *, descale_q: float, descale_k: float, descale_v: float,
                  causal: bool, scale: float, cu_seqlens=None, return_probs: bool = False):
    """Attention forward on E4M3 codes with per-tensor descales (layouts as oracle.attention)."""
    q = e4m3_decode(q8) * float(descale_q)
    k = e4m3_decode(k8) * float(descale_k)
    v = e4m3_decode(v8) * float(descale_v)
    return attention(q, k, v, causal=causal, scale=scale, cu_seqlens=cu_seqlens,
                     return_probs=return_probs)
