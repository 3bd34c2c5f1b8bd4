"""Oracle vs torch's CPU float64 scaled_dot_product_attention and logsumexp.

A library special case of the same definition: torch computes
softmax(QK^T*scale [+causal mask]) V on (B,H,S,D) tensors. No code is shared.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention, attention_rows


def _torch_ref(q, k, v, causal, scale):
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()   # (B,H,S,D)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).contiguous()
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    logits = (tq @ tk.transpose(-1, -2)) * scale
    if causal:
        S = q.shape[1]
        logits = logits.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)                          # (B,H,S)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


CASES = [
    # (config, B, H, S) reduced shapes of each workload
    ("tiny", None, None, None),
    ("mha", 1, 2, 256),
    ("mha_causal", 1, 2, 256),
    ("llama", 1, 2, 300),
    ("long", 1, 1, 384),
]


@pytest.mark.parametrize("name,B,H,S", CASES)
def test_oracle_matches_torch_sdpa(name, B, H, S):
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg, B=B, H=H, S=S)
    q, k, v = inp.f64()
    scale = float(np.float32(1.0 / np.sqrt(cfg.D)))
    o, lse = attention(q, k, v, causal=cfg.causal, scale=scale)
    ot, lt = _torch_ref(q, k, v, cfg.causal, scale)
    np.testing.assert_allclose(o, ot, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, lt, rtol=0, atol=1e-10)


def test_packed_matches_torch_per_segment():
    cfg = synth.CONFIGS["varlen"]
    lens = synth.varlen_lengths(1500, 100, 700, 99) + [0, 1]
    cu = synth.cu_seqlens_of(lens)
    T = int(cu[-1])
    q, k, v = (synth.bits_to_f64(x, "bf16") for x in synth.normal_qkv((T, 2, cfg.D), "bf16", 5))
    scale = float(np.float32(1.0 / np.sqrt(cfg.D)))
    o, lse = attention(q, k, v, causal=True, scale=scale, cu_seqlens=cu)
    for s in range(len(lens)):
        a, e = int(cu[s]), int(cu[s + 1])
        if a == e:
            continue
        ot, lt = _torch_ref(q[None, a:e], k[None, a:e], v[None, a:e], True, scale)
        np.testing.assert_allclose(o[a:e], ot[0], rtol=0, atol=1e-10)
        np.testing.assert_allclose(lse[:, a:e], lt[0], rtol=0, atol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_entry_matches_full(causal):
    q, k, v = (synth.bits_to_f64(x, "fp16") for x in synth.normal_qkv((1, 200, 3, 64), "fp16", 8))
    scale = 0.125
    o, lse = attention(q, k, v, causal=causal, scale=scale)
    rows = np.array([0, 1, 63, 64, 127, 199])
    orow, lrow = attention_rows(q[0], k[0], v[0], rows, causal=causal, scale=scale, heads=[0, 2])
    np.testing.assert_allclose(orow, o[0][rows][:, [0, 2]], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lrow, lse[0][[0, 2]][:, rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window,n_global,alibi", [(16, 0, False), (0, 5, False), (0, 0, True),
                                                   (24, 3, True), (1, 0, False), (500, 0, True)])
def test_rows_entry_matches_full_with_masks(causal, window, n_global, alibi):
    """attention_rows with the window, global-row and ALiBi variants equals the full oracle's
    rows (the full oracle's variants are pinned by brute force in test_oracle_masks.py)."""
    q, k, v = (synth.bits_to_f64(x, "bf16") for x in synth.normal_qkv((1, 230, 4, 64), "bf16", 18))
    scale = 0.125
    slopes = synth.alibi_slopes(4) if alibi else None
    o, lse = attention(q, k, v, causal=causal, scale=scale, window=window, n_global=n_global,
                       alibi_slopes=slopes)
    rows = np.array([0, 1, 2, 4, 5, 6, 63, 64, 127, 128, 200, 229])
    heads = [0, 3, 1]
    orow, lrow = attention_rows(q[0], k[0], v[0], rows, causal=causal, scale=scale, heads=heads,
                                window=window, n_global=n_global, alibi_slopes=slopes)
    np.testing.assert_allclose(orow, o[0][rows][:, heads], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lrow, lse[0][heads][:, rows], rtol=0, atol=1e-13)
