"""GPU parity of attn_bwd (dQ, dK, dV) against the fp64 backward oracle.

The GPU backward takes the GPU forward's own O and LSE; the oracle recomputes
everything from Q, K, V and dO in fp64.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import max_abs, say, scale_of, to_dev, to_f64
from oracle import attention_backward
from scaled_dot_product_08_amd import binding

pytestmark = pytest.mark.gpu

# Bound on max|g - g_ref| / max|g_ref| per gradient tensor: 4 * 2^-p with p
# the significant bits of the element type (8 for bf16, 11 for fp16). Each
# gradient passes through three 16-bit roundings of at most 2^-(p+1)
# relative each (P or dS entering the matrix product, delta from the rounded
# forward output, the stored result); sums over rows or keys partly cancel
# (dS sums to zero along a row), so the error is measured against the
# largest entry of the tensor rather than entrywise.
TOL_G = {"bf16": 4 * 2.0 ** -8, "fp16": 4 * 2.0 ** -11}


def grads(qb, kb, vb, dob, dtype, causal, scale, cu=None):
    q, k, v, do = (to_dev(x, dtype) for x in (qb, kb, vb, dob))
    cud = None if cu is None else torch.from_numpy(cu).cuda()
    o, lse = binding.fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cud)
    dq, dk, dv = binding.bwd(q, k, v, o, lse, do, causal=causal, scale=scale, cu_seqlens=cud)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(qb, kb, vb, dob, dtype, causal, scale, cu=None):
    g = grads(qb, kb, vb, dob, dtype, causal, scale, cu)
    f = [synth.bits_to_f64(x, dtype) for x in (qb, kb, vb, dob)]
    ref = attention_backward(*f, causal=causal, scale=scale, cu_seqlens=cu)
    rel = []
    for name, x, r in zip(("dq", "dk", "dv"), g, ref):
        xf = to_f64(x)
        assert np.isfinite(xf).all(), name
        m = float(np.abs(r).max())
        rel.append(max_abs(xf, r) / m if m > 0 else max_abs(xf, r))
    say(f"    rel err dq={rel[0]:.2e} dk={rel[1]:.2e} dv={rel[2]:.2e}")
    for name, e in zip(("dq", "dk", "dv"), rel):
        assert e <= TOL_G[dtype], (name, e)


SHAPES = [(1, 1, 2), (2, 33, 3), (1, 64, 2), (2, 65, 2), (1, 128, 3), (1, 129, 2), (2, 200, 2),
          (1, 333, 2), (1, 513, 1)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "bf16"), (64, "bf16"), (128, "fp16")])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{b}S{s}H{h}" for b, s, h in SHAPES])
def test_bwd_padded(shape, D, dtype, causal):
    B, S, H = shape
    say(f"bwd padded B={B} S={S} H={H} D={D} {dtype} causal={causal}")
    qb, kb, vb = synth.normal_qkv((B, S, H, D), dtype, 6000 + S)
    dob, _, _ = synth.normal_qkv((B, S, H, D), dtype, 6500 + S)
    check(qb, kb, vb, dob, dtype, causal, scale_of(D))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp16")])
def test_bwd_packed(D, dtype, causal):
    lens = [1, 3, 0, 130, 257, 64, 200, 513]
    cu = synth.cu_seqlens_of(lens)
    T, H = int(cu[-1]), 2
    say(f"bwd packed T={T} D={D} {dtype} causal={causal}")
    qb, kb, vb = synth.normal_qkv((T, H, D), dtype, 6100)
    dob, _, _ = synth.normal_qkv((T, H, D), dtype, 6101)
    check(qb, kb, vb, dob, dtype, causal, scale_of(D), cu)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.5])
def test_bwd_scale_values(scale):
    say(f"bwd scale {scale}")
    qb, kb, vb = synth.normal_qkv((1, 150, 2, 64), "fp16", 6200)
    dob, _, _ = synth.normal_qkv((1, 150, 2, 64), "fp16", 6201)
    check(qb, kb, vb, dob, "fp16", True, scale)


def test_bwd_deterministic():
    qb, kb, vb = synth.normal_qkv((2, 300, 2, 128), "bf16", 6300)
    dob, _, _ = synth.normal_qkv((2, 300, 2, 128), "bf16", 6301)
    a = grads(qb, kb, vb, dob, "bf16", True, scale_of(128))
    b = grads(qb, kb, vb, dob, "bf16", True, scale_of(128))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_llama_sampled_heads():
    """The LLaMA-shaped layer at full size; the oracle checks whole (b, h) slices."""
    cfg = synth.CONFIGS["llama"]
    say("bwd", cfg.describe())
    inp = synth.make_inputs(cfg)
    dob, _, _ = synth.normal_qkv((cfg.B, cfg.S, cfg.H, cfg.D), cfg.dtype, cfg.seed + 7)
    q, k, v, do = (to_dev(x, cfg.dtype) for x in (inp.q, inp.k, inp.v, dob))
    sc = scale_of(cfg.D)
    o, lse = binding.fwd(q, k, v, causal=True, scale=sc)
    dq, dk, dv = binding.bwd(q, k, v, o, lse, do, causal=True, scale=sc)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for b, h in [(0, 0), (3, 31), (1, 17)]:
        f = [synth.bits_to_f64(x[b:b + 1, :, h:h + 1], cfg.dtype) for x in (inp.q, inp.k, inp.v, dob)]
        ref = attention_backward(*f, causal=True, scale=sc)
        rel = []
        for x, r in zip((dq, dk, dv), ref):
            xf = x[b:b + 1, :, h:h + 1].float().numpy().astype(np.float64)
            rel.append(max_abs(xf, r) / float(np.abs(r).max()))
        say(f"    (b={b}, h={h}) rel err dq={rel[0]:.2e} dk={rel[1]:.2e} dv={rel[2]:.2e}")
        assert max(rel) <= TOL_G[cfg.dtype]
