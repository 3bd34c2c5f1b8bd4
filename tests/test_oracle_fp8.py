"""Pins of the FP8 (E4M3) oracle against torch's float8_e4m3fn and the plain oracle."""
import numpy as np
import torch

from oracle import attention, attention_fp8, e4m3_decode, e4m3_encode


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert e4m3_decode(0x7E) == 448.0 and e4m3_decode(0x01) == 2.0 ** -9
    assert e4m3_decode(0x38) == 1.0 and e4m3_decode(0xB8) == -1.0


def test_encode_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(3000) * 3, rng.standard_normal(500) * 1e-2,
                        [0.0, -0.0, 448.0, 449.0, 463.9, 464.0, 500.0, -600.0, 2.0 ** -10,
                         3 * 2.0 ** -11, 1.0625, 1.1875, 0.9375 + 2 ** -5]])
    x = x.astype(np.float32)
    mine = e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine & 0x7F, ref & 0x7F)
    fin = (ref & 0x7F) != 0x7F
    assert np.array_equal(mine[fin], ref[fin])


def test_roundtrip_of_representable_values():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_fp8_attention_is_the_plain_definition_on_decoded_inputs():
    rng = np.random.default_rng(4)
    q8, k8, v8 = (e4m3_encode(rng.standard_normal((2, 9, 2, 8))) for _ in range(3))
    o, l = attention_fp8(q8, k8, v8, descale_q=0.5, descale_k=2.0, descale_v=0.25, causal=True,
                         scale=0.3)
    qf, kf, vf = (torch.from_numpy(x).view(torch.float8_e4m3fn).double().numpy() for x in (q8, k8, v8))
    o2, l2 = attention(qf * 0.5, kf * 2.0, vf * 0.25, causal=True, scale=0.3)
    np.testing.assert_allclose(o, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l, l2, rtol=1e-14)
    # descales on Q and K act only through their product with the scale
    o3, l3 = attention_fp8(q8, k8, v8, descale_q=1.0, descale_k=1.0, descale_v=0.25, causal=True,
                           scale=0.3)
    np.testing.assert_allclose(o, o3, rtol=1e-13, atol=1e-15)
