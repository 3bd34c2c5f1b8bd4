"""GPU parity of the mask/bias variants (attn_fwd_ext): sliding window, global rows, ALiBi."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import TOL_LSE, TOL_O, max_abs, record, rne_floor, say, scale_of, to_dev, to_f64
from oracle import attention, attention_rows
from scaled_dot_product_08_amd import binding

pytestmark = pytest.mark.gpu

# Narrow windows and steep ALiBi slopes concentrate a row's weight on a few
# keys, so |O| approaches |V| (up to ~4 for N(0,1) inputs). The 16-bit output
# then carries a rounding error of up to 2^-(p+1)|O| from its own store and
# as much again from the rounded probabilities (p = 8 significant bits for
# bf16, 11 for fp16): the bound is the absolute tolerance plus 2^-p |O_ref|.
REL_O = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def run_check(qb, kb, vb, dtype, causal, scale, window, n_global, slopes, cu=None, case=None,
              tile_rows=0):
    q, k, v = to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype)
    sl = None if slopes is None else torch.from_numpy(slopes).cuda()
    cud = None if cu is None else torch.from_numpy(cu).cuda()
    o, lse = binding.fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cud, window=window,
                         n_global=n_global, alibi_slopes=sl, tile_rows=tile_rows)
    torch.cuda.synchronize()
    f = [synth.bits_to_f64(x, dtype) for x in (qb, kb, vb)]
    oref, lref = attention(*f, causal=causal, scale=scale, cu_seqlens=cu, window=window,
                           n_global=n_global, alibi_slopes=slopes)
    og = to_f64(o)
    eo, el = max_abs(og, oref), max_abs(lse.cpu().numpy(), lref)
    excess = float((np.abs(og - oref) - (TOL_O[dtype] + REL_O[dtype] * np.abs(oref))).max())
    floor = rne_floor(oref, dtype)
    say(f"    max|dO|={eo:.3e} floor={floor:.3e} max|dLSE|={el:.3e} worst excess over bound={excess:.3e}")
    if case is not None:
        record(case, dtype, eo, el, floor=floor, n_rows=int(np.prod(oref.shape[:-1])), excess=excess)
    assert excess <= 0.0, (eo, excess)
    assert el <= TOL_LSE, el


VARIANTS = [(64, 0, False), (100, 0, False), (1, 0, False), (128, 5, False), (0, 70, False),
            (0, 0, True), (200, 64, True), (33, 1, True)]


@pytest.mark.parametrize("window,n_global,alibi", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "bf16"), (64, "bf16"), (128, "fp16")])
def test_ext_padded(window, n_global, alibi, causal, D, dtype):
    B, S, H = 2, 333, 3
    say(f"ext padded S={S} D={D} {dtype} causal={causal} window={window} global={n_global} alibi={alibi}")
    qb, kb, vb = synth.normal_qkv((B, S, H, D), dtype, 4000 + window + n_global)
    run_check(qb, kb, vb, dtype, causal, scale_of(D), window, n_global,
              synth.alibi_slopes(H) if alibi else None,
              case=f"mask variant B={B} H={H} S={S} D={D} {dtype} causal={causal} window={window} "
                   f"global={n_global} alibi={alibi}")


@pytest.mark.parametrize("window,n_global,alibi", [(64, 0, False), (50, 10, True), (0, 0, True)])
@pytest.mark.parametrize("causal", [False, True])
def test_ext_packed(window, n_global, alibi, causal):
    lens = [1, 3, 0, 130, 257, 64, 200, 513]
    cu = synth.cu_seqlens_of(lens)
    T, H, D = int(cu[-1]), 2, 128
    say(f"ext packed causal={causal} window={window} global={n_global} alibi={alibi}")
    qb, kb, vb = synth.normal_qkv((T, H, D), "bf16", 4100)
    run_check(qb, kb, vb, "bf16", causal, scale_of(D), window, n_global,
              synth.alibi_slopes(H) if alibi else None, cu=cu,
              case=f"mask variant packed H={H} D={D} bf16 causal={causal} window={window} "
                   f"global={n_global} alibi={alibi}")


@pytest.mark.parametrize("S", [333, 600])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_alibi_pingpong_padded(S, causal, dtype):
    """ALiBi alone on the 8-wave ping-pong kernel (256-row tiles forced through
    attn_fwd_ext_tuned): several query and key tiles, ragged tails, against the oracle."""
    B, H, D = 2, 3, 128
    say(f"alibi ping-pong padded S={S} {dtype} causal={causal}")
    qb, kb, vb = synth.normal_qkv((B, S, H, D), dtype, 4500 + S)
    run_check(qb, kb, vb, dtype, causal, scale_of(D), 0, 0, synth.alibi_slopes(H), tile_rows=256,
              case=f"alibi ping-pong B={B} H={H} S={S} D={D} {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_alibi_pingpong_packed(causal):
    lens = [1, 3, 0, 130, 257, 64, 200, 513]
    cu = synth.cu_seqlens_of(lens)
    T, H, D = int(cu[-1]), 2, 128
    say(f"alibi ping-pong packed causal={causal}")
    qb, kb, vb = synth.normal_qkv((T, H, D), "bf16", 4600)
    run_check(qb, kb, vb, "bf16", causal, scale_of(D), 0, 0, synth.alibi_slopes(H), cu=cu,
              tile_rows=256, case=f"alibi ping-pong packed H={H} D={D} bf16 causal={causal}")


def test_alibi_layer_sampled():
    """The LLaMA-shaped layer with ALiBi, B4 H32 S4096 D128 bf16 causal, as the library runs it
    by itself (ping-pong kernel): 64 sampled rows of every (batch, head) against the oracle."""
    cfg = synth.CONFIGS["llama"]
    inp = synth.make_inputs(cfg)
    slopes = synth.alibi_slopes(cfg.H)
    say(f"alibi layer {cfg.describe()}")
    q, k, v = (to_dev(x, cfg.dtype) for x in (inp.q, inp.k, inp.v))
    o, lse = binding.fwd(q, k, v, causal=True, alibi_slopes=torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu().numpy()
    eo = el = floor = 0.0
    excess = -float("inf")
    for b in range(cfg.B):
        rows = synth.sampled_rows(cfg.S, 64, 4700 + b, must=(0, 1, 255, 256, cfg.S - 1))
        f = [synth.bits_to_f64(x[b], cfg.dtype) for x in (inp.q, inp.k, inp.v)]
        oref, lref = attention_rows(*f, rows, causal=True, scale=scale_of(cfg.D), alibi_slopes=slopes)
        og = o[b][rows].float().numpy().astype(np.float64)
        eo = max(eo, max_abs(og, oref))
        el = max(el, max_abs(lse[b][:, rows], lref))
        excess = max(excess, float((np.abs(og - oref)
                                    - (TOL_O[cfg.dtype] + REL_O[cfg.dtype] * np.abs(oref))).max()))
        floor = max(floor, rne_floor(oref, cfg.dtype))
    say(f"    sampled max|dO|={eo:.3e} floor={floor:.3e} max|dLSE|={el:.3e} excess={excess:.3e}")
    record(f"alibi layer {cfg.describe()} (64 sampled rows of every (b, h))", cfg.dtype, eo, el,
           floor=floor, n_rows=64 * cfg.B * cfg.H, excess=excess)
    assert excess <= 0.0 and el <= TOL_LSE


def test_ext_zero_slopes_match_plain():
    """Zero ALiBi slopes change nothing beyond rounding. The plain D = 64 kernel
    walks keys in 128-key tiles and the variant kernel in 64-key tiles, so the
    fp16 row sums (of rounded probabilities, 2^-11 each) are grouped
    differently; each LSE is within 2.5e-4 of exact, so they differ by <= 5e-4."""
    qb, kb, vb = synth.normal_qkv((1, 300, 2, 64), "fp16", 4200)
    q, k, v = (to_dev(x, "fp16") for x in (qb, kb, vb))
    o0, l0 = binding.fwd(q, k, v, causal=True)
    o1, l1 = binding.fwd(q, k, v, causal=True, alibi_slopes=torch.zeros(2, device="cuda"))
    torch.cuda.synchronize()
    assert (o0.float() - o1.float()).abs().max().item() <= 2e-3
    assert (l0 - l1).abs().max().item() <= 5e-4


def test_window_one_returns_v_bitwise():
    qb, kb, vb = synth.normal_qkv((2, 150, 2, 128), "bf16", 4300)
    q, k, v = (to_dev(x, "bf16") for x in (qb, kb, vb))
    o, _ = binding.fwd(q, k, v, causal=True, window=1)
    torch.cuda.synchronize()
    assert torch.equal(o, v)


def test_long_window_global_sampled():
    """The pages' long-context scheme: window 4096 plus 64 global query rows, B1 H32 S65536 D128;
    96 sampled rows (global, window-edge and interior ones) of every head."""
    S, H, D, W, G = 65536, 32, 128, 4096, 64
    say(f"window workload S={S} H={H} D={D} window={W} global={G}")
    qb, kb, vb = synth.normal_qkv((1, S, H, D), "bf16", 4400)
    q, k, v = (to_dev(x, "bf16") for x in (qb, kb, vb))
    o, lse = binding.fwd(q, k, v, causal=True, window=W, n_global=G)
    torch.cuda.synchronize()
    rows = synth.sampled_rows(S, 96, 4401, must=(0, 1, 63, 64, 65, 4095, 4096, 4097, S - 1))
    o, lse = o.cpu(), lse.cpu()
    eo = el = floor = 0.0
    excess = -float("inf")
    for h0 in range(0, H, 8):
        heads = list(range(h0, h0 + 8))
        f = [synth.bits_to_f64(x[0][:, heads], "bf16") for x in (qb, kb, vb)]
        oref, lref = attention_rows(*f, rows, causal=True, scale=scale_of(D), window=W, n_global=G)
        og = o[0][rows][:, heads].float().numpy().astype(np.float64)
        eo = max(eo, max_abs(og, oref))
        el = max(el, max_abs(lse[0][heads][:, rows].numpy(), lref))
        excess = max(excess, float((np.abs(og - oref)
                                    - (TOL_O["bf16"] + REL_O["bf16"] * np.abs(oref))).max()))
        floor = max(floor, rne_floor(oref, "bf16"))
    say(f"    sampled max|dO|={eo:.3e} floor={floor:.3e} max|dLSE|={el:.3e} excess={excess:.3e}")
    record(f"mask variant B=1 H={H} S={S} D={D} bf16 causal window={W} global={G} "
           f"(96 sampled rows of every head)", "bf16", eo, el, floor=floor, n_rows=len(rows) * H,
           excess=excess)
    assert excess <= 0.0 and el <= TOL_LSE
