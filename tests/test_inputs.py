"""Seeded generator: determinism, rounding, packing metadata."""
import numpy as np
import torch

import synth


def test_same_seed_same_bytes():
    a = synth.make_inputs(synth.CONFIGS["tiny"])
    b = synth.make_inputs(synth.CONFIGS["tiny"])
    assert a.sha256 == b.sha256
    c = synth.make_inputs(synth.CONFIGS["mha"], B=1, H=1, S=64)
    assert c.sha256 != a.sha256


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0]   # exact ties
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_fp16_and_decode_roundtrip():
    x = np.random.default_rng(1).standard_normal(5000).astype(np.float32)
    bits = synth.f32_to_fp16_bits(x)
    np.testing.assert_array_equal(synth.bits_to_f64(bits, "fp16"), x.astype(np.float16).astype(np.float64))
    bb = synth.f32_to_bf16_bits(x)
    back = synth.bits_to_f64(bb, "bf16")
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


def test_varlen_lengths_recipe():
    lens = synth.varlen_lengths(65536, 128, 8192, synth.CONFIGS["varlen"].seed + 1)
    assert sum(lens) == 65536
    assert all(128 <= n <= 8192 for n in lens[:-1])
    assert 1 <= lens[-1] <= 8192
    cu = synth.cu_seqlens_of(lens)
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == 65536 and np.all(np.diff(cu) >= 0)


def test_sampled_rows_recipe():
    rows = synth.sampled_rows(65536, 256, synth.CONFIGS["long"].seed + 2)
    assert len(rows) == 256 and len(set(rows.tolist())) == 256
    for r in (0, 1, 63, 64, 127, 128, 65535):
        assert r in rows


def test_llama_scale_factor_exact():
    q, _, _ = synth.normal_qkv((1, 8, 2, 16), "bf16", 5, mult=0.5)
    q1, _, _ = synth.normal_qkv((1, 8, 2, 16), "bf16", 5, mult=1.0)
    np.testing.assert_array_equal(synth.bits_to_f64(q, "bf16") * 2, synth.bits_to_f64(q1, "bf16"))
