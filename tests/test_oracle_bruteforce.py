"""Oracle vs pure-Python brute force on tiny inputs (relative 1e-12)."""
import numpy as np
import pytest

import bruteforce
import synth
from oracle import attention


def _inputs(shape, dtype, seed):
    q, k, v = synth.normal_qkv(shape, dtype, seed)
    return (synth.bits_to_f64(q, dtype), synth.bits_to_f64(k, dtype), synth.bits_to_f64(v, dtype))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,H,D", [(1, 1, 1, 1), (2, 5, 2, 3), (1, 16, 2, 8), (2, 9, 1, 8)])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_padded_matches_bruteforce(B, S, H, D, causal, dtype):
    q, k, v = _inputs((B, S, H, D), dtype, 11 + B * 100 + S)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o, lse = attention(q, k, v, causal=causal, scale=scale)
    ob, lb = bruteforce.padded(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    ob = np.array(ob)
    lb = np.array(lb)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lb, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_matches_bruteforce(causal):
    lens = [1, 3, 0, 5]
    cu = synth.cu_seqlens_of(lens)
    T, H, D = int(cu[-1]), 2, 8
    q, k, v = _inputs((T, H, D), "bf16", 7)
    scale = 0.37
    o, lse = attention(q, k, v, causal=causal, scale=scale, cu_seqlens=cu)
    ob, lb = bruteforce.packed(q.tolist(), k.tolist(), v.tolist(), cu.tolist(), causal, scale)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12, atol=1e-14)


def test_bruteforce_catches_planted_mistakes():
    """Each plausible oracle mistake, planted in a copy of the arithmetic, fails the brute-force pin."""
    q, k, v = _inputs((1, 6, 1, 4), "fp16", 3)
    scale = 0.5
    ob, lb = bruteforce.padded(q.tolist(), k.tolist(), v.tolist(), True, scale)
    ob = np.array(ob)[0, :, 0]
    qh, kh, vh = q[0, :, 0], k[0, :, 0], v[0, :, 0]

    def variant(kind):
        s = (qh @ kh.T) * (1.0 if kind == "noscale" else scale)
        if kind == "transposed":
            s = s.T
        allowed = np.tril(np.ones((6, 6), bool), -1 if kind == "strict_causal" else 0)
        s = np.where(allowed, s, -np.inf)
        m = s.max(1)
        w = np.exp(s - m[:, None]) if kind != "signflip" else np.exp(-(s - m[:, None]))
        w = np.where(np.isfinite(w), w, 0.0)
        w[~allowed] = 0.0
        p = w / w.sum(1)[:, None]
        return p @ vh

    for kind in ("noscale", "transposed", "strict_causal", "signflip"):
        with np.errstate(all="ignore"):
            bad = variant(kind)
        assert not np.allclose(bad, ob, rtol=1e-6, atol=1e-9), kind
