"""Pins of the KV-cache decode oracle (oracle/decode.py) against independent references."""
import math

import numpy as np
import pytest
import torch

import bruteforce
from oracle import attention, decode_attention


def rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,S_max,lens", [(1, 7, [7, 3, 0]), (3, 6, [6, 2, 5]), (2, 5, [1, 5, 4])])
def test_decode_matches_bruteforce(causal, Sq, S_max, lens):
    B, H, D = len(lens), 2, 3
    q = rand((B, Sq, H, D), 1)
    kc = rand((B, H, S_max, D), 2)
    vc = rand((B, H, S_max, D + 1), 3)
    o, lse = decode_attention(q, kc, vc, causal=causal, scale=0.7, seqlens_k=lens)
    ob, lb = bruteforce.decode(q.tolist(), kc.tolist(), vc.tolist(), lens, causal, 0.7)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-13)
    lb = np.array(lb)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_torch_sdpa(causal):
    B, Sq, H, D, S_max = 3, 4, 2, 16, 40
    lens = [40, 17, 4]
    q = rand((B, Sq, H, D), 4)
    kc = rand((B, H, S_max, D), 5)
    vc = rand((B, H, S_max, D), 6)
    o, lse = decode_attention(q, kc, vc, causal=causal, scale=0.25, seqlens_k=lens)
    for b, L in enumerate(lens):
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)[None]          # (1, H, Sq, D)
        kt = torch.from_numpy(kc[b, :, :L])[None]
        vt = torch.from_numpy(vc[b, :, :L])[None]
        pos = torch.arange(Sq)[:, None] + (L - Sq)
        mask = (torch.arange(L)[None, :] <= pos) if causal else torch.ones(Sq, L, dtype=torch.bool)
        ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.25)
        np.testing.assert_allclose(o[b], ot[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
        lt = torch.logsumexp((qt @ kt.transpose(-1, -2) * 0.25).masked_fill(~mask, -math.inf), -1)
        np.testing.assert_allclose(lse[b], lt[0].numpy(), rtol=1e-10)


def test_full_length_causal_decode_is_the_causal_forward():
    """Sq = L under causality: every token of the sequence is a query; the
    result is the causal forward of those L tokens (the (B,S,H,D) form)."""
    B, H, L, D = 2, 3, 9, 8
    q = rand((B, L, H, D), 7)
    k = rand((B, L, H, D), 8)
    v = rand((B, L, H, D), 9)
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    o1, l1 = decode_attention(q, kc, vc, causal=True, scale=0.4)
    o2, l2 = attention(q, k, v, causal=True, scale=0.4)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


def test_single_row_is_last_row_of_the_noncausal_forward():
    B, H, L, D, S_max = 1, 2, 12, 4, 20
    k = rand((B, S_max, H, D), 10)
    v = rand((B, S_max, H, D), 11)
    q = rand((B, L, H, D), 12)
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    o1, l1 = decode_attention(q[:, -1:], kc, vc, causal=True, scale=0.3, seqlens_k=[L])
    o2, l2 = attention(q, k[:, :L], v[:, :L], causal=False, scale=0.3)
    np.testing.assert_allclose(o1[:, 0], o2[:, -1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1[:, :, 0], l2[:, :, -1], rtol=1e-12)


def test_closed_forms_and_empty_rows():
    q = rand((2, 2, 1, 4), 13)
    kc = rand((2, 1, 5, 4), 14)
    vc = rand((2, 1, 5, 4), 15)
    # sequence 0 holds one key: the non-causal rows return V[0] and LSE = scale q.k0
    o, lse = decode_attention(q, kc, vc, causal=False, scale=0.5, seqlens_k=[1, 0])
    np.testing.assert_allclose(o[0, :, 0], np.repeat(vc[0, 0, :1], 2, axis=0), rtol=1e-15)
    np.testing.assert_allclose(lse[0, 0], 0.5 * q[0, :, 0] @ kc[0, 0, 0], rtol=1e-14)
    # sequence 1 holds none: zeros and -inf
    assert (o[1] == 0).all() and np.isneginf(lse[1]).all()
    # causal with one key and two rows: row 0 sits before the cache start and sees nothing
    o, lse = decode_attention(q, kc, vc, causal=True, scale=0.5, seqlens_k=[1, 5])
    assert (o[0, 0] == 0).all() and np.isneginf(lse[0, 0, 0])
    np.testing.assert_allclose(o[0, 1, 0], vc[0, 0, 0], rtol=1e-15)


def test_keys_past_the_valid_length_are_ignored():
    q = rand((1, 1, 2, 8), 16)
    kc = rand((1, 2, 10, 8), 17)
    vc = rand((1, 2, 10, 8), 18)
    o1, l1 = decode_attention(q, kc, vc, causal=False, scale=0.3, seqlens_k=[6])
    kc[:, :, 6:] = 1e3
    vc[:, :, 6:] = np.nan
    o2, l2 = decode_attention(q, kc, vc, causal=False, scale=0.3, seqlens_k=[6])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_misaligned_causal_mask_is_caught():
    """The brute-force pin separates the end-aligned mask from a start-aligned one."""
    B, Sq, H, D, L = 1, 3, 1, 4, 6
    q = rand((B, Sq, H, D), 19)
    kc = rand((B, H, L, D), 20)
    vc = rand((B, H, L, D), 21)
    ob, _ = bruteforce.decode(q.tolist(), kc.tolist(), vc.tolist(), [L], True, 0.5)
    # start-aligned: row i sees keys 0..i
    wrong = np.zeros((Sq, D))
    for i in range(Sq):
        s = kc[0, 0, :i + 1] @ q[0, i, 0] * 0.5
        w = np.exp(s - s.max())
        wrong[i] = (w / w.sum()) @ vc[0, 0, :i + 1]
    assert np.abs(wrong - np.array(ob)[0, :, 0]).max() > 1e-3
