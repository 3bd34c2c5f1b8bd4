"""Closed-form invariants the oracle must satisfy (mathematics, not the oracle itself)."""
import math

import numpy as np
import pytest

import synth
from oracle import attention


def _rand(shape, seed, dtype="fp16"):
    return tuple(synth.bits_to_f64(x, dtype) for x in synth.normal_qkv(shape, dtype, seed))


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    q, k, v = _rand((2, 33, 2, 16), 1)
    _, _, probs = attention(q, k, v, causal=causal, scale=0.25, return_probs=True)
    for p in probs.values():
        assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-12)
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("how", ["q0", "k0", "scale0"])
def test_equal_scores_give_mean_of_v(causal, how):
    q, k, v = _rand((1, 40, 2, 8), 2)
    scale = 0.3
    if how == "q0":
        q[:] = 0
    elif how == "k0":
        k[:] = 0
    else:
        scale = 0.0
    o, lse = attention(q, k, v, causal=causal, scale=scale)
    S = q.shape[1]
    for i in range(S):
        n = i + 1 if causal else S
        np.testing.assert_allclose(o[0, i], v[0, :n].mean(axis=0), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=0, atol=1e-12)


def test_causal_row0_returns_v0():
    q, k, v = _rand((2, 17, 3, 8), 3)
    scale = 0.7
    o, lse = attention(q, k, v, causal=True, scale=scale)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])
    expect = scale * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], expect, rtol=0, atol=1e-13)


def test_kv_permutation_invariance_noncausal():
    q, k, v = _rand((1, 50, 2, 8), 4)
    perm = np.random.default_rng(0).permutation(50)
    o1, l1 = attention(q, k, v, causal=False, scale=0.4)
    o2, l2 = attention(q, k[:, perm], v[:, perm], causal=False, scale=0.4)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    """An extra feature with q=1, k=c adds c*scale to every score of a row: O unchanged, LSE shifts."""
    q, k, v = _rand((1, 30, 1, 8), 5)
    scale, c = 0.5, 3.0
    q2 = np.concatenate([q, np.ones(q.shape[:-1] + (1,))], axis=-1)
    k2 = np.concatenate([k, np.full(k.shape[:-1] + (1,), c)], axis=-1)
    o1, l1 = attention(q, k, v, causal=causal, scale=scale)
    o2, l2 = attention(q2, k2, v, causal=causal, scale=scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, c * scale, rtol=0, atol=1e-12)


def test_huge_scale_selects_argmax():
    q, k, v = _rand((1, 20, 1, 8), 6)
    o, _ = attention(q, k, v, causal=False, scale=1e4)
    s = q[0, :, 0] @ k[0, :, 0].T
    np.testing.assert_allclose(o[0, :, 0], v[0, s.argmax(axis=1), 0], rtol=0, atol=1e-9)


def test_last_causal_row_equals_noncausal_last_row():
    q, k, v = _rand((1, 25, 2, 8), 7)
    oc, lc = attention(q, k, v, causal=True, scale=0.3)
    on, ln = attention(q, k, v, causal=False, scale=0.3)
    np.testing.assert_allclose(oc[0, -1], on[0, -1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lc[0, :, -1], ln[0, :, -1], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_separate_calls(causal):
    lens = [5, 0, 12, 1, 7]
    cu = synth.cu_seqlens_of(lens)
    q, k, v = _rand((int(cu[-1]), 2, 8), 8, "bf16")
    o, lse = attention(q, k, v, causal=causal, scale=0.35, cu_seqlens=cu)
    for s in range(len(lens)):
        a, e = cu[s], cu[s + 1]
        if a == e:
            continue
        os_, ls_ = attention(q[None, a:e], k[None, a:e], v[None, a:e], causal=causal, scale=0.35)
        np.testing.assert_array_equal(o[a:e], os_[0])
        np.testing.assert_array_equal(lse[:, a:e], ls_[0])


def test_head_and_batch_permutation_commute():
    q, k, v = _rand((3, 12, 4, 8), 9)
    o, lse = attention(q, k, v, causal=True, scale=0.3)
    hp, bp = [2, 0, 3, 1], [1, 2, 0]
    o2, l2 = attention(q[bp][:, :, hp], k[bp][:, :, hp], v[bp][:, :, hp], causal=True, scale=0.3)
    np.testing.assert_array_equal(o2, o[bp][:, :, hp])
    np.testing.assert_array_equal(l2, lse[bp][:, hp])


def test_integer_structure_counts():
    """Q=K=0: exp(LSE) recovers the number of visible keys exactly."""
    lens = [3, 9, 1]
    cu = synth.cu_seqlens_of(lens)
    T = int(cu[-1])
    q = np.zeros((T, 1, 4)); k = np.zeros((T, 1, 4))
    v = np.repeat(np.array([1.0, 2.0, 3.0]), lens)[:, None, None] * np.ones((T, 1, 4))
    o, lse = attention(q, k, v, causal=True, scale=0.5, cu_seqlens=cu)
    counts = np.rint(np.exp(lse[0])).astype(int)
    expect = np.concatenate([np.arange(1, n + 1) for n in lens])
    np.testing.assert_array_equal(counts, expect)
    np.testing.assert_allclose(o[:, 0, 0], np.repeat([1.0, 2.0, 3.0], lens), rtol=0, atol=1e-14)
