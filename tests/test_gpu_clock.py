"""attn_clock_sample: the per-CU shader-clock and real-time counters it records advance, and
their ratio over a sustained attention workload is a plausible shader clock."""
import pytest
import torch

import synth
from gpu_util import say, to_dev
from scaled_dot_product_08_amd import binding

pytestmark = pytest.mark.gpu


def test_clock_counters_advance_and_give_a_plausible_clock():
    st = torch.cuda.current_stream()
    n = 2 * binding.CLOCK_SLOTS
    buf = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    qb, kb, vb = synth.normal_qkv((2, 2048, 8, 128), "bf16", 41)
    q, k, v = (to_dev(x, "bf16") for x in (qb, kb, vb))
    binding.fwd(q, k, v, causal=True)            # warm the kernel up
    e0, e1 = torch.cuda.Event(), torch.cuda.Event()
    e0.record(st)                                  # barrier before each sample
    binding.clock_sample(buf[:n], st)
    for _ in range(50):
        binding.fwd(q, k, v, causal=True)
    e1.record(st)
    binding.clock_sample(buf[n:], st)
    torch.cuda.synchronize()
    c = buf.cpu().tolist()
    per = sorted(binding.clock_mhz(c[:n], c[n:]))
    say(f"    {len(per)} CUs: shader clock min {per[0]:.0f} median {per[len(per) // 2]:.0f} "
        f"max {per[-1]:.0f} MHz")
    assert len(per) >= 200, "most CUs ran a sampling wave in both samples"
    assert 100.0 < per[len(per) // 2] < 3000.0
