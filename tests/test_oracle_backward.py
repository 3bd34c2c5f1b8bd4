"""Pins of the backward oracle (oracle/backward.py) against independent references."""
import numpy as np
import pytest
import torch

from oracle import attention, attention_backward


def rand(shape, seed, s=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * s


def loss(q, k, v, do, causal, scale, cu=None):
    o, _ = attention(q, k, v, causal=causal, scale=scale, cu_seqlens=cu)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    """Central differences of the (separately pinned) forward oracle."""
    B, S, H, D = 1, 5, 2, 3
    q, k, v, do = rand((B, S, H, D), 1), rand((B, S, H, D), 2), rand((B, S, H, D), 3), rand((B, S, H, D), 4)
    scale = 0.6
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = loss(args["q"], args["k"], args["v"], do, causal, scale)
            args[name] = xm
            fm = loss(args["q"], args["k"], args["v"], do, causal, scale)
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    B, S, H, D = 2, 37, 3, 16
    q, k, v, do = (rand((B, S, H, D), 10 + i) for i in range(4))
    scale = 0.25
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).clone().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(g, t.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-9, atol=1e-11)


def test_backward_closed_forms():
    B, S, H, D = 2, 9, 2, 4
    q, k, v, do = (rand((B, S, H, D), 20 + i) for i in range(4))
    for causal in (False, True):
        dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=0.7)
        # each softmax row sums to one: dK sums to zero over the keys, dV to the sum of dO
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), rtol=1e-12, atol=1e-12)
    # zero scale: uniform rows, no gradient reaches q or k
    dq, dk, dv = attention_backward(q, k, v, do, causal=False, scale=0.0)
    assert not dq.any() and not dk.any()
    np.testing.assert_allclose(dv, np.repeat(do.mean(axis=1, keepdims=True), S, axis=1), rtol=1e-12)
    # causal, key S-1 is seen only by row S-1 with weight p_{S-1,S-1}
    dq, dk, dv = attention_backward(q, k, v, do, causal=True, scale=0.7)
    s = 0.7 * np.einsum("bhd,bshd->bhs", q[:, -1], k)
    p_last = np.exp(s - s.max(-1, keepdims=True))
    p_last = p_last[..., -1] / p_last.sum(-1)
    np.testing.assert_allclose(dv[:, -1], p_last[..., None] * do[:, -1], rtol=1e-12)


def test_backward_packed_equals_per_sequence():
    lens = [3, 0, 6, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, D = int(cu[-1]), 2, 5
    q, k, v, do = (rand((T, H, D), 30 + i) for i in range(4))
    g = attention_backward(q, k, v, do, causal=True, scale=0.4, cu_seqlens=cu)
    for a, e in zip(cu[:-1], cu[1:]):
        if e == a:
            continue
        gs = attention_backward(q[None, a:e], k[None, a:e], v[None, a:e], do[None, a:e], causal=True,
                                scale=0.4)
        for x, y in zip(g, gs):
            np.testing.assert_allclose(x[a:e], y[0], rtol=1e-13, atol=1e-15)


def test_planted_transpose_is_caught():
    """A dK computed as dS Q (missing transpose) fails the finite-difference pin."""
    S, D = 4, 3
    q, k, v, do = (rand((1, S, 1, D), 40 + i) for i in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, causal=False, scale=0.5)
    s = 0.5 * q[0, :, 0] @ k[0, :, 0].T
    p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    dp = do[0, :, 0] @ v[0, :, 0].T
    ds = p * (dp - (p * dp).sum(1, keepdims=True))
    wrong = 0.5 * ds @ q[0, :, 0]
    assert np.abs(wrong - dk[0, :, 0]).max() > 1e-3
