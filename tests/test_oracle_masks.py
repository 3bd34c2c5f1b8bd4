"""Pins of the oracle's mask/bias variants: sliding window + global rows, ALiBi."""
import numpy as np
import pytest
import torch

import bruteforce
import synth
from oracle import attention
from oracle.attention import visible_mask


def _rand(shape, seed, dtype="fp16"):
    return tuple(synth.bits_to_f64(x, dtype) for x in synth.normal_qkv(shape, dtype, seed))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window,n_global", [(1, 0), (3, 0), (4, 2), (0, 3), (2, 9)])
@pytest.mark.parametrize("alibi", [False, True])
def test_masks_match_bruteforce(causal, window, n_global, alibi):
    q, k, v = _rand((2, 9, 2, 4), 31 + window + 7 * n_global)
    scale = 0.4
    slopes = [0.5, 0.125] if alibi else None
    o, lse = attention(q, k, v, causal=causal, scale=scale, window=window, n_global=n_global,
                       alibi_slopes=slopes)
    ob, lb = bruteforce.padded_ext(q.tolist(), k.tolist(), v.tolist(), causal, scale, window,
                                   n_global, slopes)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_masks_match_torch_float_mask(causal):
    """torch's fp64 SDPA with an explicit additive float mask (bias, -inf where hidden)."""
    q, k, v = _rand((1, 200, 3, 16), 5, "bf16")
    scale, window, n_global = 0.25, 37, 5
    slopes = np.array([0.3, 0.05, 0.0])
    o, lse = attention(q, k, v, causal=causal, scale=scale, window=window, n_global=n_global,
                       alibi_slopes=slopes)
    S = q.shape[1]
    vis = visible_mask(np.arange(S), S, causal, window, n_global)
    dist = np.abs(np.arange(S)[:, None] - np.arange(S)[None, :])
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    for h in range(3):
        bias = np.where(vis, -slopes[h] * dist, -np.inf)
        mask = torch.from_numpy(bias)[None, None]
        ot = torch.nn.functional.scaled_dot_product_attention(tq[:, h:h + 1], tk[:, h:h + 1], tv[:, h:h + 1],
                                                              attn_mask=mask, scale=scale)
        lt = torch.logsumexp((tq[:, h:h + 1] @ tk[:, h:h + 1].transpose(-1, -2)) * scale + mask, dim=-1)
        np.testing.assert_allclose(o[:, :, h], ot[:, 0].numpy(), rtol=0, atol=1e-10)
        np.testing.assert_allclose(lse[:, h], lt[:, 0].numpy(), rtol=0, atol=1e-10)


def test_wide_window_equals_plain_and_zero_slopes_equal_no_bias():
    q, k, v = _rand((1, 40, 2, 8), 6)
    for causal in (False, True):
        o0, l0 = attention(q, k, v, causal=causal, scale=0.3)
        o1, l1 = attention(q, k, v, causal=causal, scale=0.3, window=40, alibi_slopes=[0.0, 0.0])
        np.testing.assert_array_equal(o0, o1)
        np.testing.assert_array_equal(l0, l1)


def test_all_rows_global_is_full_attention():
    q, k, v = _rand((1, 30, 2, 8), 7)
    o0, l0 = attention(q, k, v, causal=False, scale=0.3)
    o1, l1 = attention(q, k, v, causal=True, scale=0.3, window=3, n_global=30)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_window_one_returns_own_value():
    q, k, v = _rand((2, 25, 2, 8), 8)
    o, lse = attention(q, k, v, causal=True, scale=0.7, window=1)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.7 * np.einsum("bshd,bshd->bhs", q, k), rtol=0, atol=1e-13)


def test_steep_alibi_concentrates_on_the_diagonal():
    q, k, v = _rand((1, 20, 1, 8), 9)
    o, _ = attention(q, k, v, causal=True, scale=0.1, alibi_slopes=[200.0])
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-30 + 1e-12)
