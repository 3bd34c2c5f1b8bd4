"""attn_clock_sample: the shader-clock and real-time counters it records advance, and their
ratio over a sustained attention workload is a plausible shader clock."""
import pytest
import torch

import synth
from gpu_util import say, to_dev
from scaled_dot_product_08_amd import binding

pytestmark = pytest.mark.gpu


def test_clock_counters_advance_and_give_a_plausible_clock():
    st = torch.cuda.current_stream()
    buf = torch.zeros(4, dtype=torch.int64, device="cuda")
    qb, kb, vb = synth.normal_qkv((2, 2048, 8, 128), "bf16", 41)
    q, k, v = (to_dev(x, "bf16") for x in (qb, kb, vb))
    binding.fwd(q, k, v, causal=True)            # warm the kernel up
    binding.clock_sample(buf[0:2], st)
    for _ in range(50):
        binding.fwd(q, k, v, causal=True)
    binding.clock_sample(buf[2:4], st)
    torch.cuda.synchronize()
    c = buf.cpu().tolist()
    cycles, ticks = c[2] - c[0], c[3] - c[1]
    mhz = cycles / ticks * 100.0
    say(f"    {cycles} shader cycles over {ticks} ticks of 100 MHz: {mhz:.0f} MHz")
    assert cycles > 0 and ticks > 0
    assert 100.0 < mhz < 3000.0
