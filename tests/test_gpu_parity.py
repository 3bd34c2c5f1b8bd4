"""GPU parity: the HIP library (through the C ABI) against the fp64 CPU oracle.

Bar: max-abs error on O within 4e-3 (fp16) / 1e-2 (bf16), on LSE within 1e-3,
element by element on the same seeded inputs.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import TOL_LSE, TOL_O, max_abs, record, rne_floor, say, scale_of, to_dev, to_f64
from oracle import attention, attention_rows
from scaled_dot_product_08_amd import binding

pytestmark = pytest.mark.gpu


def run_padded(qb, kb, vb, dtype, causal, scale, with_lse=True, shape=(0, 0)):
    q, k, v = to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype)
    o, lse = binding.fwd(q, k, v, causal=causal, scale=scale, with_lse=with_lse,
                         tile_rows=shape[0], key_split=shape[1])
    torch.cuda.synchronize()
    return o, lse


def check_full(qb, kb, vb, dtype, causal, scale, cu=None, shape=(0, 0), case=None):
    """Whole-output comparison (small shapes); ``case`` names the recorded margins."""
    qf, kf, vf = (synth.bits_to_f64(x, dtype) for x in (qb, kb, vb))
    if cu is None:
        o, lse = run_padded(qb, kb, vb, dtype, causal, scale, shape=shape)
        oref, lref = attention(qf, kf, vf, causal=causal, scale=scale)
    else:
        q, k, v = to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype)
        cud = torch.from_numpy(cu).cuda()
        o, lse = binding.fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cud,
                             tile_rows=shape[0], key_split=shape[1])
        torch.cuda.synchronize()
        oref, lref = attention(qf, kf, vf, causal=causal, scale=scale, cu_seqlens=cu)
    eo, el = max_abs(to_f64(o), oref), max_abs(lse.cpu().numpy(), lref)
    say(f"    max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    if case is not None:
        record(case, dtype, eo, el, oref=oref, n_rows=int(np.prod(oref.shape[:-1])))
    assert eo <= TOL_O[dtype], eo
    assert el <= TOL_LSE, el
    return eo, el


# ---- the five workloads -------------------------------------------------------

def test_config_tiny():
    cfg = synth.CONFIGS["tiny"]
    say("tiny", cfg.describe())
    inp = synth.make_inputs(cfg)
    check_full(inp.q, inp.k, inp.v, cfg.dtype, cfg.causal, scale_of(cfg.D),
               case="tiny " + cfg.describe() + " (every output)")


@pytest.mark.parametrize("name", ["mha", "mha_causal"])
def test_config_mha_full(name):
    cfg = synth.CONFIGS[name]
    say(name, cfg.describe())
    inp = synth.make_inputs(cfg)
    check_full(inp.q, inp.k, inp.v, cfg.dtype, cfg.causal, scale_of(cfg.D),
               case=name + " " + cfg.describe() + " (every output)")


@pytest.mark.parametrize("wg", [(128, 2), (256, 1)], ids=["bm128ks2", "bm256"])
@pytest.mark.parametrize("name", ["mha", "mha_causal"])
def test_config_mha_full_other_shapes(name, wg):
    """The B=4 H=12 S=2048 D=64 workloads with the workgroup shapes the size heuristic does
    not pick for them (the key split and 256-row tiles), every output against the oracle."""
    cfg = synth.CONFIGS[name]
    say(name, cfg.describe(), "shape", wg)
    inp = synth.make_inputs(cfg)
    check_full(inp.q, inp.k, inp.v, cfg.dtype, cfg.causal, scale_of(cfg.D), shape=wg)


def _sampled_padded(cfg, rows_per_head, heads_stride=1, seed_off=2, case=None):
    inp = synth.make_inputs(cfg)
    scale = scale_of(cfg.D)
    o, lse = run_padded(inp.q, inp.k, inp.v, cfg.dtype, cfg.causal, scale)
    o = o.cpu()
    lse = lse.cpu().numpy()
    worst_o = worst_l = floor = 0.0
    n_rows = 0
    for b in range(cfg.B):
        rows = synth.sampled_rows(cfg.S, rows_per_head, cfg.seed + seed_off + b)
        heads = list(range(0, cfg.H, heads_stride))
        qf, kf, vf = (synth.bits_to_f64(x[b], cfg.dtype) for x in (inp.q, inp.k, inp.v))
        oref, lref = attention_rows(qf, kf, vf, rows, causal=cfg.causal, scale=scale, heads=heads)
        og = o[b][rows][:, heads].float().numpy().astype(np.float64)
        worst_o = max(worst_o, max_abs(og, oref))
        worst_l = max(worst_l, max_abs(lse[b][heads][:, rows], lref))
        floor = max(floor, rne_floor(oref, cfg.dtype))
        n_rows += len(rows) * len(heads)
    say(f"    sampled max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e} ({n_rows} rows)")
    if case is not None:
        record(case, cfg.dtype, worst_o, worst_l, floor=floor, n_rows=n_rows)
    assert worst_o <= TOL_O[cfg.dtype]
    assert worst_l <= TOL_LSE
    assert torch.isfinite(o.float()).all()


def test_config_llama_sampled():
    """256 sampled query rows of every (batch, head) of the LLaMA-shaped layer, each against
    all the keys it sees."""
    cfg = synth.CONFIGS["llama"]
    say("llama", cfg.describe())
    _sampled_padded(cfg, rows_per_head=256,
                    case="llama " + cfg.describe() + " (256 sampled rows of every (b, h))")


def test_config_long_sampled():
    cfg = synth.CONFIGS["long"]
    say("long", cfg.describe())
    _sampled_padded(cfg, rows_per_head=cfg.sample_rows, heads_stride=1,
                    case=f"long {cfg.describe()} ({cfg.sample_rows} sampled rows of every head)")


def test_config_varlen_sampled():
    cfg = synth.CONFIGS["varlen"]
    say("varlen", cfg.describe())
    inp = synth.make_inputs(cfg)
    cu = inp.cu_seqlens
    scale = scale_of(cfg.D)
    q, k, v = to_dev(inp.q, cfg.dtype), to_dev(inp.k, cfg.dtype), to_dev(inp.v, cfg.dtype)
    o, lse = binding.fwd(q, k, v, causal=True, scale=scale, cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    o = o.cpu()
    lse = lse.cpu().numpy()
    say(f"    {len(cu) - 1} segments, lengths {np.diff(cu).tolist()}")
    worst_o = worst_l = floor = 0.0
    n_rows = 0
    heads = list(range(cfg.H))
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        L = e - a
        rows = synth.sampled_rows(L, min(L, 64), cfg.seed + 2 + s)
        qf, kf, vf = (synth.bits_to_f64(x[a:e], cfg.dtype) for x in (inp.q, inp.k, inp.v))
        oref, lref = attention_rows(qf, kf, vf, rows, causal=True, scale=scale, heads=heads)
        og = o[a:e][rows][:, heads].float().numpy().astype(np.float64)
        worst_o = max(worst_o, max_abs(og, oref))
        worst_l = max(worst_l, max_abs(lse[heads][:, a + rows], lref))
        floor = max(floor, rne_floor(oref, cfg.dtype))
        n_rows += len(rows) * len(heads)
    say(f"    sampled max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e} ({n_rows} rows)")
    record(f"varlen {cfg.describe()} (64 sampled rows of every sequence, all {cfg.H} heads)",
           cfg.dtype, worst_o, worst_l, floor=floor, n_rows=n_rows)
    assert worst_o <= TOL_O[cfg.dtype]
    assert worst_l <= TOL_LSE
    assert torch.isfinite(o.float()).all()


# ---- reduced shapes: every tile boundary, ragged tails, both dtypes / D ----------

SHAPES = [
    (1, 1, 1), (1, 2, 2), (2, 3, 63), (1, 2, 64), (1, 2, 65), (2, 2, 127), (1, 3, 128),
    (1, 2, 129), (2, 1, 200), (1, 2, 255), (1, 1, 256), (1, 2, 300), (1, 1, 517),
]


SHAPE_PARAMS = [(128, 1), (128, 2), (256, 1)]
SHAPE_IDS = ["bm128", "bm128ks2", "bm256"]


@pytest.fixture(params=SHAPE_PARAMS, ids=SHAPE_IDS)
def shape(request):
    """Run the test with each workgroup shape: 128-row tiles (4 waves), 128-row tiles whose
    keys two groups of 4 waves split, and 256-row tiles (8 waves)."""
    return request.param


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,S", SHAPES)
def test_padded_shapes(B, H, S, D, dtype, causal, shape):
    say(f"padded B={B} H={H} S={S} D={D} {dtype} causal={causal} shape={shape}")
    qb, kb, vb = synth.normal_qkv((B, S, H, D), dtype, 1000 + S + D)
    check_full(qb, kb, vb, dtype, causal, scale_of(D), shape=shape)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_shapes(D, dtype, causal, shape):
    lens = [1, 3, 0, 130, 257, 64, 0, 128, 200, 513]
    cu = synth.cu_seqlens_of(lens)
    T = int(cu[-1])
    say(f"packed lens={lens} D={D} {dtype} causal={causal} shape={shape}")
    qb, kb, vb = synth.normal_qkv((T, 3, D), dtype, 77 + D)
    check_full(qb, kb, vb, dtype, causal, scale_of(D), cu=cu, shape=shape)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9, 3.0])
def test_scale_values(scale):
    say(f"scale={scale}")
    qb, kb, vb = synth.normal_qkv((1, 150, 2, 64), "fp16", 5)
    check_full(qb, kb, vb, "fp16", True, scale)
    check_full(qb, kb, vb, "fp16", False, scale)


def test_lse_optional():
    qb, kb, vb = synth.normal_qkv((1, 130, 2, 128), "bf16", 6)
    o1, _ = run_padded(qb, kb, vb, "bf16", True, 0.1)
    o2, l2 = run_padded(qb, kb, vb, "bf16", True, 0.1, with_lse=False)
    assert l2 is None
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("name", ["llama", "mha_causal", "mha"])
def test_tile_size_choice(name):
    """Workgroup shapes against each other. 128- and 256-row query tiles: bitwise identical O
    and LSE (same per-row arithmetic over the same 64-key tiles). The key split adds two
    partial sums, so its lazy maximum and row sums are grouped differently: each result is
    within the oracle tolerance, hence they differ by at most twice it (O) and by 5e-4 (LSE,
    twice the 2.5e-4 bound of the fp16 row sums)."""
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg, B=2 if cfg.B > 2 else cfg.B)
    outs = []
    for shape in SHAPE_PARAMS:
        o, lse = run_padded(inp.q, inp.k, inp.v, cfg.dtype, cfg.causal, scale_of(cfg.D),
                            shape=shape)
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[0][1], outs[2][1])
    for a in range(len(outs)):
        for b in range(a + 1, len(outs)):
            assert (outs[a][0].float() - outs[b][0].float()).abs().max().item() <= 2 * TOL_O[cfg.dtype]
            assert (outs[a][1] - outs[b][1]).abs().max().item() <= 5e-4


def test_page_s2050_ragged_case():
    """The ragged S=2050 shape the pages single out (tail tile of 2 rows)."""
    qb, kb, vb = synth.normal_qkv((1, 2050, 2, 64), "fp16", 2050)
    check_full(qb, kb, vb, "fp16", False, scale_of(64))
    check_full(qb, kb, vb, "fp16", True, scale_of(64))


def _ramp_qkv(B, S, H, D, dtype, step, seed, jump_every=0):
    """Scores that climb along the key axis: every key row is (base + step * j) * u
    for one unit direction u shared with the queries, plus small noise; with
    jump_every > 0 the climb happens in steps at every jump_every-th key instead.
    Later key tiles then exceed any maximum taken on earlier ones, which drives
    the kernel's maximum refresh (and, for small steps, its acceptance of a stale
    maximum) on every tile."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    j = np.arange(S, dtype=np.float64)
    if jump_every:
        j = np.floor(j / jump_every) * jump_every
    q = np.broadcast_to(u, (B, S, H, D)) * 2.0 + 0.1 * rng.standard_normal((B, S, H, D))
    k = (1.0 + step * j)[None, :, None, None] * u + 0.1 * rng.standard_normal((B, S, H, D))
    v = rng.standard_normal((B, S, H, D))
    return tuple(synth.to_bits(x.astype(np.float32), dtype) for x in (q, k, v))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("step,jump", [(0.05, 0), (0.12, 32), (0.4, 64), (1.0, 64)])
@pytest.mark.parametrize("wg", [(0, 0), (256, 1)], ids=["auto", "bm256"])
def test_climbing_scores_refresh_the_maximum(dtype, D, causal, step, jump, wg):
    """Keys whose scores keep rising (linearly, or in jumps at tile and half-tile
    boundaries): the running maximum is stale on almost every tile, by amounts
    both below and far above the refresh thresholds. O and LSE stay within the
    oracle tolerance. With 256-row tiles the 8-wave instances (for D = 128 the ping-pong
    schedule) find the bound broken after their first tile and walk their keys again."""
    S = 333
    qb, kb, vb = _ramp_qkv(1, S, 2, D, dtype, step, seed=91 + D + int(100 * step), jump_every=jump)
    say(f"climb dtype={dtype} D={D} causal={causal} step={step} jump={jump} shape={wg}")
    check_full(qb, kb, vb, dtype, causal, scale_of(D), shape=wg)
