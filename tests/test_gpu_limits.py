"""GPU parity at the edges of the accepted sizes: the largest head count, a very long single
sequence, and a decode cache of 4M rows (32-bit byte offsets within one (batch, head) slice)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import TOL_LSE, TOL_O, max_abs, say, scale_of, to_dev, to_f64
from oracle import attention, attention_rows, decode_attention
from scaled_dot_product_08_amd import binding

pytestmark = pytest.mark.gpu


def test_max_heads():
    """H = 65535 (the largest accepted): token stride 65535 * D elements, 65535 workgroups."""
    B, S, H, D = 1, 3, 65535, 64
    say(f"max heads B={B} S={S} H={H} D={D}")
    qb, kb, vb = synth.normal_qkv((B, S, H, D), "fp16", 8000)
    q, k, v = (to_dev(x, "fp16") for x in (qb, kb, vb))
    o, lse = binding.fwd(q, k, v, causal=True, scale=scale_of(D))
    torch.cuda.synchronize()
    heads = [0, 1, 4097, 32768, 65534]
    f = [synth.bits_to_f64(x[:, :, heads], "fp16") for x in (qb, kb, vb)]
    oref, lref = attention(*f, causal=True, scale=scale_of(D))
    eo = max_abs(to_f64(o[:, :, heads]), oref)
    el = max_abs(lse[:, heads].cpu().numpy(), lref)
    say(f"    max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O["fp16"] and el <= TOL_LSE


@pytest.mark.parametrize("tile_rows", [128, 256])
def test_max_heads_d128_full_tiles(tile_rows):
    """H = 65535 at D = 128 with whole 128/256-row query tiles: a tile spans up to
    256 * 65535 * 256 bytes, 64 KB under 2^32, the largest byte range a buffer descriptor of
    the kernel covers. Four heads carry seeded inputs and are checked against the oracle; every
    other head has Q = K = V = 0, so its output must be exactly 0 and exp(LSE) the count of
    visible keys (i + 1 under causality), which checks every head's tile mapping and offsets."""
    B, S, H, D = 1, 256, 65535, 128
    say(f"max heads D=128 B={B} S={S} H={H} tile_rows={tile_rows}")
    q = torch.zeros((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    heads = [0, 1, 32768, 65534]
    qb, kb, vb = synth.normal_qkv((B, S, len(heads), D), "bf16", 8050)
    for i, h in enumerate(heads):
        q[:, :, h] = to_dev(np.ascontiguousarray(qb[:, :, i]), "bf16")
        k[:, :, h] = to_dev(np.ascontiguousarray(kb[:, :, i]), "bf16")
        v[:, :, h] = to_dev(np.ascontiguousarray(vb[:, :, i]), "bf16")
    o, lse = binding.fwd(q, k, v, causal=True, scale=scale_of(D), tile_rows=tile_rows,
                         key_split=2 if tile_rows == 128 else 1)
    torch.cuda.synchronize()
    f = [synth.bits_to_f64(x, "bf16") for x in (qb, kb, vb)]
    oref, lref = attention(*f, causal=True, scale=scale_of(D))
    eo = max_abs(to_f64(o[:, :, heads]), oref)
    el = max_abs(lse[:, heads].cpu().numpy(), lref)
    say(f"    seeded heads max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE
    zero = torch.ones(H, dtype=torch.bool, device="cuda")
    zero[heads] = False
    assert (o[:, :, zero] == 0).all().item()
    counts = torch.exp(lse[:, zero].double()).round()
    expect = torch.arange(1, S + 1, dtype=torch.float64, device="cuda")
    assert (counts == expect).all().item()


def test_long_single_sequence():
    """One 262144-token sequence, one head, causal: 2048 query tiles of one (b, h)."""
    B, S, H, D = 1, 262144, 1, 64
    say(f"long sequence S={S}")
    qb, kb, vb = synth.normal_qkv((B, S, H, D), "bf16", 8100)
    q, k, v = (to_dev(x, "bf16") for x in (qb, kb, vb))
    o, lse = binding.fwd(q, k, v, causal=True, scale=scale_of(D))
    torch.cuda.synchronize()
    rows = synth.sampled_rows(S, 24, 8101, must=(0, 1, 127, 128, 131071, 131072, S - 2))
    f = [synth.bits_to_f64(x[0], "bf16") for x in (qb, kb, vb)]
    oref, lref = attention_rows(*f, rows, causal=True, scale=scale_of(D))
    eo = max_abs(o[0].cpu()[rows].float().numpy(), oref)
    el = max_abs(lse[0].cpu()[:, rows].numpy(), lref)
    say(f"    sampled max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE


@pytest.mark.parametrize("num_splits", [0, 1])
def test_decode_4m_cache(num_splits):
    """A 4M-row cache (512 MB per tensor at D = 64): byte offsets up to 2^29 in one slice."""
    B, Sq, H, S_max, D = 1, 1, 1, 1 << 22, 64
    say(f"decode S_max={S_max} splits={num_splits}")
    inp = synth.decode_inputs(B, Sq, H, S_max, D, "fp16", 8200, [S_max - 5])
    q, k, v = (to_dev(x, "fp16") for x in (inp.q, inp.k, inp.v))
    sl = torch.from_numpy(inp.seqlens).cuda()
    o, lse = binding.decode(q, k, v, seqlens_k=sl, scale=scale_of(D), num_splits=num_splits)
    torch.cuda.synchronize()
    f = [synth.bits_to_f64(x, "fp16") for x in (inp.q, inp.k, inp.v)]
    oref, lref = decode_attention(*f, causal=False, scale=scale_of(D), seqlens_k=inp.seqlens)
    eo = max_abs(to_f64(o), oref)
    el = max_abs(lse.cpu().numpy(), lref)
    say(f"    max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O["fp16"] and el <= TOL_LSE
