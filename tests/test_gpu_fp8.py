"""GPU parity of attn_fwd_fp8 (E4M3 Q, K, V) against the fp64 FP8 oracle.

Bound per output element, derived from the arithmetic: the probabilities
enter P V as E4M3 codes of P * 2^4, which round to nearest with at most
2^-4 relative error when P * 2^4 is a normal E4M3 value, and at most 2^-14
absolute error (half the subnormal step, divided by 2^4) below that, i.e.
for probabilities under 2^-10 of the row maximum. Hence
    |O - O_ref| <= 2^-4 (P |V|) + 2^-14 (M |V|) + 2^-(p+1) |O_ref| + 1e-5
with P the oracle's probabilities, M marking the visible keys whose
probability is below 2^-10 of the row's largest, and p the output type's
significant bits (8 bf16, 11 fp16). The LSE sums fp32 probabilities and
keeps the 16-bit path's 1e-3.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import TOL_LSE, max_abs, say, scale_of, to_f64
from oracle import attention_fp8, e4m3_decode, e4m3_encode
from oracle.attention import _head_rows, visible_mask
from scaled_dot_product_08_amd import binding

pytestmark = pytest.mark.gpu

OUT = {"bf16": (torch.bfloat16, 8), "fp16": (torch.float16, 11)}


def u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def head_bound(P, Vabs, Oref, causal, bits):
    L = P.shape[1]
    vis = visible_mask(np.arange(P.shape[0]), L, causal)
    rowmax = P.max(axis=1, keepdims=True)
    small = vis & (P < rowmax * 2.0 ** -10)
    return (2.0 ** -4 * (P @ Vabs) + 2.0 ** -14 * (small.astype(np.float64) @ Vabs)
            + 2.0 ** -(bits + 1) * np.abs(Oref) + 1e-5)


def check(q8, k8, v8, causal, scale, dsc, out, cu=None):
    dq, dk, dv = dsc
    tdt, bits = OUT[out]
    cud = None if cu is None else torch.from_numpy(cu).cuda()
    o, lse = binding.fwd_fp8(u8(q8), u8(k8), u8(v8), causal=causal, scale=scale, descale_q=dq,
                             descale_k=dk, descale_v=dv, out_dtype=tdt, cu_seqlens=cud)
    torch.cuda.synchronize()
    oref, lref, probs = attention_fp8(q8, k8, v8, descale_q=dq, descale_k=dk, descale_v=dv,
                                      causal=causal, scale=scale, cu_seqlens=cu, return_probs=True)
    vabs = np.abs(e4m3_decode(v8) * dv)
    og = to_f64(o)
    bound = np.zeros_like(oref)
    if cu is None:
        for (b, h), P in probs.items():
            bound[b, :, h] = head_bound(P, vabs[b, :, h], oref[b, :, h], causal, bits)
    else:
        for (si, h), P in probs.items():
            a, e = int(cu[si]), int(cu[si + 1])
            bound[a:e, h] = head_bound(P, vabs[a:e, h], oref[a:e, h], causal, bits)
    err = np.abs(og - oref)
    el = max_abs(lse.cpu().numpy(), lref)
    say(f"    max|dO|={err.max():.3e} max err/bound={float((err / bound).max()):.3f} "
        f"max|dLSE|={el:.3e}")
    assert (err <= bound).all()
    assert el <= TOL_LSE


SHAPES = [(1, 1, 2), (2, 33, 3), (1, 64, 2), (2, 65, 2), (1, 128, 2), (1, 129, 2), (2, 200, 2),
          (1, 333, 2), (1, 513, 1)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("out", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{b}S{s}H{h}" for b, s, h in SHAPES])
def test_fp8_padded(shape, out, causal):
    B, S, H = shape
    say(f"fp8 padded B={B} S={S} H={H} out={out} causal={causal}")
    q8, k8, v8 = synth.fp8_qkv((B, S, H, 128), 7000 + S)
    check(q8, k8, v8, causal, scale_of(128), (1.0, 1.0, 1.0), out)


@pytest.mark.parametrize("dsc", [(0.5, 0.25, 2.0), (2.0, 1.0, 0.125), (-1.0, 0.5, 1.0), (0.0, 1.0, 1.0)])
def test_fp8_descales(dsc):
    say(f"fp8 descales {dsc}")
    q8, k8, v8 = synth.fp8_qkv((2, 150, 2, 128), 7100)
    check(q8, k8, v8, True, scale_of(128), dsc, "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_packed(causal):
    lens = [1, 3, 0, 130, 257, 64, 200, 513]
    cu = synth.cu_seqlens_of(lens)
    T = int(cu[-1])
    say(f"fp8 packed T={T} causal={causal}")
    q8, k8, v8 = synth.fp8_qkv((T, 2, 128), 7200)
    check(q8, k8, v8, causal, scale_of(128), (1.0, 1.0, 1.0), "bf16", cu)


def test_fp8_llama_shape_sampled():
    """B4 H32 S4096 D128 causal with E4M3 inputs (the LLaMA-shaped layer), sampled rows."""
    B, S, H, D = 4, 4096, 32, 128
    say(f"fp8 B={B} S={S} H={H}")
    q8, k8, v8 = synth.fp8_qkv((B, S, H, D), 7300, mult=0.5)
    o, lse = binding.fwd_fp8(u8(q8), u8(k8), u8(v8), causal=True, scale=scale_of(D))
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    rows = synth.sampled_rows(S, 24, 7301)
    worst = 0.0
    worst_l = 0.0
    for b, h in [(0, 0), (3, 31), (2, 9)]:
        qf, kf, vf = (e4m3_decode(x[b, :, h]) for x in (q8, k8, v8))
        oref, lref, P = _head_rows(qf, kf, vf, rows, True, scale_of(D))
        Lk = P.shape[1]
        vis = visible_mask(rows, Lk, True)
        small = vis & (P < P.max(axis=1, keepdims=True) * 2.0 ** -10)
        bound = (2.0 ** -4 * (P @ np.abs(vf)) + 2.0 ** -14 * (small @ np.abs(vf))
                 + 2.0 ** -9 * np.abs(oref) + 1e-5)
        err = np.abs(o[b, rows, h].float().numpy().astype(np.float64) - oref)
        worst = max(worst, float((err / bound).max()))
        worst_l = max(worst_l, max_abs(lse[b, h, rows].numpy(), lref))
    say(f"    sampled max err/bound={worst:.3f} max|dLSE|={worst_l:.3e}")
    assert worst <= 1.0 and worst_l <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("step,jump", [(0.02, 0), (0.1, 32), (0.08, 64)])
def test_fp8_climbing_scores(step, jump, causal):
    """Key scores that climb along the keys (linearly, or in jumps at 32- and 64-key
    boundaries): the running maximum is stale on almost every tile, by amounts below
    and far above what the kernel accepts without a refresh (every P * 2^4 must stay
    within the E4M3 range). Same bound as the other cases."""
    S, H, D = 333, 2, 128
    rng = np.random.default_rng(7300 + int(100 * step) + jump)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    j = np.arange(S, dtype=np.float64)
    if jump:
        j = np.floor(j / jump) * jump
    q = np.broadcast_to(u, (1, S, H, D)) * 4.0 + 0.1 * rng.standard_normal((1, S, H, D))
    k = (1.0 + step * j)[None, :, None, None] * u * 4.0 + 0.1 * rng.standard_normal((1, S, H, D))
    v = rng.standard_normal((1, S, H, D))
    q8, k8, v8 = (e4m3_encode(x) for x in (q, k, v))
    say(f"fp8 climbing step={step} jump={jump} causal={causal}")
    check(q8, k8, v8, causal, scale_of(D), (1.0, 1.0, 1.0), "bf16")
