"""Attention-forward benchmark: TFLOP/s and fraction of MI355X dense MFMA peak.

One step = one call of the fused attention forward (the whole hot path: one
kernel launch) over one batch of synthetic input already resident in HBM.
Default workload: the LLaMA-2-7B-shaped layer, B=4 H=32 S=4096 D=128 bf16
causal (Q/K/V ~ N(0,1)*0.5). Prints ONE JSON line.

Timing: W untimed warm-up launches, then a settle phase of untimed launches
(--settle-ms of GPU work; the chip's power management runs the shader clock
low for the first tens of milliseconds after the GPU has been idle), then
exactly K launches timed with HIP events on the launch stream. The host does
not wait between the settle launches and the timed ones, so the GPU runs from
one into the other without idling. The average
shader clock over the timed loop comes from the GPU's own counters (the
library's attn_clock_sample, enqueued right before and after the timed
launches); socket power is sampled with amdsmi over the settle phase and the
timed loop.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MFMA peak (B4 H12 S2048 D64 fp16; S4096 D128 bf16)"
PEAK_TFLOPS = 2516.6          # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E peak bandwidth
PEAK_TFLOPS_FP8 = 5033.2      # MI355X dense fp8 MFMA: twice the fp16/bf16 rate
KERNEL_SOURCES = ["scaled_dot_product_08_amd/csrc/attn_fwd_kernel.hip",
                  "scaled_dot_product_08_amd/csrc/attn_kernel.h",
                  "scaled_dot_product_08_amd/csrc/gfx950_util.h"]
DECODE_SOURCES = ["scaled_dot_product_08_amd/csrc/attn_decode_kernel.hip",
                  "scaled_dot_product_08_amd/csrc/attn_decode.h",
                  "scaled_dot_product_08_amd/csrc/gfx950_util.h"]


# The pages' own attention-forward figures, for context only (other hardware):
# NVIDIA A100 SXM4 40GB (312 TFLOP/s dense FP16 tensor peak), CUDA 12.1,
# PyTorch 2.2, FP16, sequence length 2048, head dimension 64
# (jianying88.com/news/49672 §1 and §4.3).
PAGES_CONTEXT = {
    "hardware": "NVIDIA A100 SXM4 40GB, CUDA 12.1, PyTorch 2.2 (312 TFLOP/s FP16 peak)",
    "workload": "attention forward, FP16, seq_len 2048, head_dim 64 (batch not stated)",
    "unfused_tflops": 42,
    "fused_tflops": 287,
    "fused_tflops_at_seq_len_2050": 213,
    "source": "jianying88.com/news/49672 §1, §4.3",
    "note": "context on other hardware, not a target",
}


class ClockSampler:
    """Samples the GPU's shader clock (MHz, per XCD) and socket power (W) with amdsmi
    from a background thread; ``window(t0, t1)`` summarises the samples taken between
    two host times."""

    def __init__(self, period_s: float = 0.002):
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:          # no amdsmi / no permission: report why
            self._smi = None
            self.error = repr(e)

    def start(self):
        if self._smi is None:
            return self
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def _run(self):
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and c > 0]
                pw = m.get("current_socket_power")
                self.samples.append((time.perf_counter(), m.get("current_gfxclk"), clks,
                                     pw if isinstance(pw, (int, float)) else None))
            except Exception as e:
                self.error = repr(e)
                return
            time.sleep(self.period)

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def window(self, t0: float, t1: float):
        """amdsmi readings between two host times (its metrics refresh slowly: a
        window of tens of milliseconds may hold stale values)."""
        if self._smi is None:
            return {"available": False, "error": self.error}
        sel = [x for x in self.samples if t0 <= x[0] <= t1]
        if not sel:
            return {"available": True, "samples": 0}
        per_xcd = [c for x in sel for c in x[2]] or [x[1] for x in sel if isinstance(x[1], int)]
        pw = [x[3] for x in sel if x[3] is not None]
        return {"available": True, "samples": len(sel),
                "amdsmi_sclk_mhz_mean": round(sum(per_xcd) / len(per_xcd), 1),
                "socket_power_w_mean": round(sum(pw) / len(pw), 1) if pw else None}


CLOCK = None     # the ClockSampler of this run (set in main)


def peak_at(mhz):
    """Dense fp16/bf16 MFMA peak at a shader clock: 256 CU x 4096 FLOP/clk x f."""
    if not mhz:
        return None
    return round(256 * 4096 * mhz * 1e6 / 1e12, 1)


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in (sources or KERNEL_SOURCES):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_INPUTS = {}


def inputs_of(cfg):
    """Seeded inputs of a workload, kept for the oracle timings of the same run (except the
    128K-token one, which is large and not timed on the host)."""
    import synth
    if cfg.name in _INPUTS:
        return _INPUTS[cfg.name]
    inp = synth.make_inputs(cfg)
    if cfg.S * cfg.B <= 65536:
        _INPUTS[cfg.name] = inp
    return inp


def make_device_inputs(cfg):
    import numpy as np
    import torch

    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    inp = inputs_of(cfg)
    dev = [torch.from_numpy(x.view(np.int16)).view(dt).cuda() for x in (inp.q, inp.k, inp.v)]
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).cuda()
    return inp, dev, cu


def settle(step, settle_ms: float, per_launch_ms: float):
    """Untimed launches until about ``settle_ms`` of GPU work has been enqueued. The host
    waits for every chunk but the last, so the GPU goes from the settle launches straight
    into whatever is enqueued next, with no idle gap: after even a short idle period the
    power management brings the shader clock back up over the next tens of milliseconds."""
    import torch
    if settle_ms <= 0:
        return {"launches": 0, "ms_of_gpu_work": 0.0, "host_wait_before_timing": True}
    n = 0
    chunk = max(1, int(20.0 / max(per_launch_ms, 1e-3)))      # ~20 ms per chunk
    target = max(1, int(settle_ms / max(per_launch_ms, 1e-3)))
    while n < target:
        if n:
            torch.cuda.synchronize()
        for _ in range(min(chunk, target - n)):
            step()
        n += min(chunk, target - n)
    return {"launches": n, "ms_of_gpu_work": round(n * per_launch_ms, 1),
            "host_wait_before_timing": False}


def timed(step, steps: int, warmup: int, settle_ms: float, stream):
    """warmup launches, a settle phase, then ``steps`` launches between two HIP events
    on ``stream``; returns (ms per launch, settle record, clock record)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    step()
    torch.cuda.synchronize()
    hs = time.perf_counter()
    per_launch_ms = (hs - t_w) * 1e3
    # Everything the timed region needs is allocated before the settle launches,
    # so nothing between them and the timed loop can wait for the device.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    pre = torch.cuda.Event(enable_timing=True)
    from scaled_dot_product_08_amd import binding
    n = 2 * binding.CLOCK_SLOTS
    ctr = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    st = settle(step, settle_ms, per_launch_ms)
    pre.record(stream)                     # barrier: the settle launches have finished
    binding.clock_sample(ctr[:n], stream)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)                      # barrier: the timed launches have finished
    binding.clock_sample(ctr[n:], stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    c = ctr.cpu().tolist()
    per = sorted(binding.clock_mhz(c[:n], c[n:]))
    clock = {"sclk_mhz": round(per[len(per) // 2], 1) if per else None,
             "cus": len(per),
             "sclk_mhz_min": round(per[0], 1) if per else None,
             "sclk_mhz_max": round(per[-1], 1) if per else None,
             "source": "median over CUs of each CU's shader-clock counter over the timed loop "
                       "(attn_clock_sample)"}
    if CLOCK is not None:
        clock["settle_and_timed"] = CLOCK.window(hs, h1)
    return t0.elapsed_time(t1) / steps, st, clock


def time_workload(cfg, steps: int, warmup: int, samples: int = 0, settle_ms: float = 0.0,
                  tile_rows: int = 0, key_split: int = 0, head_group: int = 0):
    """Mean over ``steps`` back-to-back launches bracketed by events (after ``warmup``
    launches and a settle phase of ``settle_ms``); with ``samples``, also that many
    individually timed launches afterwards (median and minimum)."""
    import numpy as np
    import torch

    import synth
    from scaled_dot_product_08_amd import accounting, binding

    inp, (q, k, v), cu = make_device_inputs(cfg)
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))
    out = torch.empty_like(q)
    if cu is None:
        lse = torch.empty((cfg.B, cfg.H, cfg.S), dtype=torch.float32, device="cuda")
        if cfg.window or cfg.n_global:
            fl = accounting.masked_flops(cfg.B, cfg.H, cfg.S, cfg.D, cfg.causal, cfg.window,
                                         cfg.n_global)
        else:
            fl = accounting.flops(cfg.B, cfg.H, cfg.S, cfg.D, cfg.causal)
        nbytes = accounting.min_hbm_bytes(cfg.B, cfg.H, cfg.S, cfg.D, cfg.dtype)
    else:
        lse = torch.empty((cfg.H, cfg.S), dtype=torch.float32, device="cuda")
        lens = np.diff(inp.cu_seqlens)
        fl = accounting.varlen_flops(lens, cfg.H, cfg.D, cfg.causal)
        nbytes = accounting.min_hbm_bytes(1, cfg.H, cfg.S, cfg.D, cfg.dtype)
    stream = torch.cuda.current_stream()
    slopes = torch.from_numpy(synth.alibi_slopes(cfg.H)).cuda() if cfg.alibi else None

    def step():
        binding.attn_fwd(q, k, v, out, lse, causal=cfg.causal, scale=scale, cu_seqlens=cu,
                         stream=stream, window=cfg.window, n_global=cfg.n_global,
                         alibi_slopes=slopes, tile_rows=tile_rows, key_split=key_split,
                         head_group=head_group)

    ms, st, clk = timed(step, steps, warmup, settle_ms, stream)
    res = {"ms": ms, "flops": fl, "bytes": nbytes, "tflops": fl / (ms * 1e-3) / 1e12,
           "sha256": inp.sha256, "settle": st, "clock": clk}
    if samples > 0:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(samples)]
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        res["per_launch_us"] = {"samples": samples, "median": round(per[len(per) // 2], 2),
                                "min": round(per[0], 2)}
    return res


def device_peak():
    """CUs x 4096 FLOP/clk x the device's maximum shader clock, from the HIP runtime."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        cus, khz = ctypes.c_int(0), ctypes.c_int(0)
        # hipDeviceAttributeMultiprocessorCount = 63, hipDeviceAttributeClockRate = 5 (kHz)
        if hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, 0) != 0:
            return None
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0) != 0:
            return None
        return {"cus": cus.value, "max_sclk_mhz": khz.value / 1e3,
                "tflops": round(cus.value * 4096 * khz.value * 1e3 / 1e12, 1)}
    except OSError:
        return None


def time_fp8(cfg, steps: int, warmup: int, settle_ms: float = 0.0):
    """attn_fwd_fp8 on E4M3 inputs of a forward workload's shape (bf16 output)."""
    import numpy as np
    import torch

    import synth
    from scaled_dot_product_08_amd import accounting, binding

    q8, k8, v8 = (torch.from_numpy(x).cuda()
                  for x in synth.fp8_qkv((cfg.B, cfg.S, cfg.H, cfg.D), cfg.seed + 9, cfg.mult))
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((cfg.B, cfg.H, cfg.S), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fl = accounting.flops(cfg.B, cfg.H, cfg.S, cfg.D, cfg.causal)

    def step():
        st = binding.attn_fwd_fp8_raw(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                                      lse.data_ptr(), cfg.B, cfg.H, cfg.S, cfg.D, int(cfg.causal),
                                      scale, 1.0, 1.0, 1.0, binding.ATTN_DTYPE_BF16, None,
                                      stream.cuda_stream)
        if st != 0:
            raise binding.AttnError(st, binding.attn_strerror(st))

    ms, st, clk = timed(step, steps, warmup, settle_ms, stream)
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": cfg.describe().replace(cfg.dtype, "e4m3 (bf16 out)"),
            "us_per_call": round(ms * 1e3, 2), "tflops": round(tf, 1),
            "frac_of_fp8_peak": round(tf / PEAK_TFLOPS_FP8, 4), "settle": st, "clock": clk}


def time_backward(cfg, steps: int, warmup: int, settle_ms: float = 0.0):
    """attn_bwd over a forward workload: mean over ``steps`` launches of both kernels."""
    import numpy as np
    import torch

    import synth
    from scaled_dot_product_08_amd import accounting, binding

    inp, (q, k, v), cu = make_device_inputs(cfg)
    dt = q.dtype
    dob, _, _ = synth.normal_qkv(inp.q.shape, cfg.dtype, cfg.seed + 7)
    do = torch.from_numpy(dob.view(np.int16)).view(dt).cuda()
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))
    o, lse = binding.fwd(q, k, v, causal=cfg.causal, scale=scale, cu_seqlens=cu)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B = cfg.B if cu is None else cu.numel() - 1
    ws = torch.empty(binding.bwd_workspace_size(B, cfg.H, cfg.S, cu is not None), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    if cu is None:
        fl = accounting.flops(cfg.B, cfg.H, cfg.S, cfg.D, cfg.causal)
    else:
        fl = accounting.varlen_flops(np.diff(inp.cu_seqlens), cfg.H, cfg.D, cfg.causal)
    fl *= accounting.BACKWARD_FLOP_RATIO

    def step():
        binding.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, causal=cfg.causal, scale=scale,
                         cu_seqlens=cu, workspace=ws, stream=stream)

    ms, st, clk = timed(step, steps, warmup, settle_ms, stream)
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": "backward " + cfg.describe(), "us_per_call": round(ms * 1e3, 2),
            "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS, 4), "settle": st,
            "clock": clk}


def time_decode(cfg, steps: int, warmup: int, settle_ms: float = 0.0):
    """KV-cache decode step: mean over ``steps`` launches, inputs resident in HBM."""
    import numpy as np
    import torch

    import synth
    from scaled_dot_product_08_amd import accounting, binding

    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    inp = synth.make_decode_inputs(cfg)
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(dt).cuda() for x in (inp.q, inp.k, inp.v))
    sl = None if inp.seqlens is None else torch.from_numpy(inp.seqlens).cuda()
    lens = [cfg.S_max] * cfg.B if inp.seqlens is None else inp.seqlens.tolist()
    out = torch.empty_like(q)
    lse = torch.empty((cfg.B, cfg.H, cfg.Sq), dtype=torch.float32, device="cuda")
    ws_bytes = binding.decode_workspace_size(cfg.B, cfg.H, cfg.Sq, cfg.S_max, cfg.D, 0)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))
    stream = torch.cuda.current_stream()

    def step():
        binding.attn_decode(q, k, v, out, lse, seqlens_k=sl, causal=cfg.causal, scale=scale,
                            workspace=ws, stream=stream)

    ms, st, clk = timed(step, steps, warmup, settle_ms, stream)
    nbytes = accounting.decode_bytes(cfg.B, cfg.H, cfg.Sq, cfg.D, lens, cfg.dtype)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": cfg.describe(), "us_per_call": round(ms * 1e3, 2),
            "algorithmic_bytes": nbytes, "GB_per_s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "tflops": round(accounting.decode_flops(cfg.H, cfg.Sq, cfg.D, lens) / (ms * 1e-3) / 1e12, 2),
            "traffic": read_traffic(cfg.name, DECODE_SOURCES),
            "kernel_source": kernel_source_hash(DECODE_SOURCES), "settle": st, "clock": clk}


def read_traffic(workload: str, sources=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return rec.get("traffic_bytes_per_launch")


def _host_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        return None


def _oracle_time(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def oracle_config_timing(name: str, max_s: float = 4.0):
    """The fp64 oracle (as it stands) on one workload, on this host's cores.

    Whole workload where that takes seconds; otherwise a bounded sample of it (whole
    (sequence, head) slices, or the sampled query rows the parity tests use), with the
    full-workload time extrapolated by the ratio of oracle work (score entries it
    materialises) and labelled so."""
    import numpy as np

    import synth
    from oracle import attention, attention_rows
    from scaled_dot_product_08_amd import accounting

    cfg = synth.CONFIGS[name]
    inp = inputs_of(cfg)
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))
    f64 = lambda x: synth.bits_to_f64(x, cfg.dtype)
    rec = {"workload": cfg.describe()}
    if cfg.varlen:
        cu = inp.cu_seqlens
        lens = np.diff(cu)
        order = np.argsort(lens)[::-1]
        done, dt, entries = [], 0.0, 0.0
        # whole (sequence, head) slices, longest sequences first, until the budget is spent
        for s_idx in order:
            a, e = int(cu[s_idx]), int(cu[s_idx + 1])
            qs, ks, vs = (f64(x[a:e]) for x in (inp.q, inp.k, inp.v))
            for h in range(cfg.H):
                dt += _oracle_time(lambda: attention(qs[None, :, h:h + 1], ks[None, :, h:h + 1],
                                                     vs[None, :, h:h + 1], causal=cfg.causal,
                                                     scale=scale))
                entries += float(e - a) ** 2
                done.append((int(s_idx), h))
                if dt >= max_s:
                    break
            if dt >= max_s:
                break
        full_entries = float(cfg.H) * float((lens.astype(np.float64) ** 2).sum())
        rec.update({"sample": f"{len(done)} whole (sequence, head) slices of the "
                              f"{len(lens)} x {cfg.H}, longest sequences first",
                    "seconds": round(dt, 2),
                    "extrapolated_full_seconds": round(dt * full_entries / entries, 1)})
    elif cfg.sample_rows:
        b = 0
        rows = synth.sampled_rows(cfg.S, cfg.sample_rows, cfg.seed + 2 + b)
        qb, kb, vb = (f64(x[b]) for x in (inp.q, inp.k, inp.v))
        dt, heads = 0.0, 0
        for h in range(cfg.H):
            dt += _oracle_time(lambda: attention_rows(qb, kb, vb, rows, causal=cfg.causal,
                                                      scale=scale, heads=[h]))
            heads += 1
            if dt >= max_s:
                break
        kmax = int(rows.max()) + 1 if cfg.causal else cfg.S
        sample_entries = heads * len(rows) * float(kmax)
        full_entries = cfg.B * cfg.H * float(cfg.S) ** 2
        rec.update({"sample": f"{len(rows)} sampled query rows (the parity rows) of {heads} of "
                              f"{cfg.H} heads",
                    "seconds": round(dt, 2),
                    "extrapolated_parity_sample_seconds": round(dt * cfg.H / heads, 1),
                    "extrapolated_full_seconds": round(dt * full_entries / sample_entries, 1)})
    else:
        # whole (batch, head) slices until the budget is spent
        dt, n = 0.0, 0
        for b in range(cfg.B):
            qb, kb, vb = (f64(x[b:b + 1]) for x in (inp.q, inp.k, inp.v))
            for h in range(cfg.H):
                dt += _oracle_time(lambda: attention(qb[:, :, h:h + 1], kb[:, :, h:h + 1],
                                                     vb[:, :, h:h + 1], causal=cfg.causal,
                                                     scale=scale))
                n += 1
                if dt >= max_s:
                    break
            if dt >= max_s:
                break
        total = cfg.B * cfg.H
        rec.update({"sample": ("the whole workload" if n == total else
                               f"{n} of the {total} whole (batch, head) slices"),
                    "seconds": round(dt, 2),
                    "tflops": round(accounting.flops(1, n, cfg.S, cfg.D, cfg.causal) / dt / 1e12, 4)})
        if n < total:
            rec["extrapolated_full_seconds"] = round(dt * total / n, 1)
    return rec


def cpu_baseline(cfg, budget_s: float = 15.0):
    """The fp64 oracle on whole (batch, head) slices of the headline workload (every row
    against every key it sees), for about ``budget_s`` on this host's cores."""
    import numpy as np

    import synth
    from oracle import attention
    from scaled_dot_product_08_amd import accounting

    cores = len(os.sched_getaffinity(0))
    inp = inputs_of(cfg)
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))
    dt, n = 0.0, 0
    for b in range(cfg.B):
        qb, kb, vb = (synth.bits_to_f64(x[b:b + 1], cfg.dtype) for x in (inp.q, inp.k, inp.v))
        for h in range(cfg.H):
            dt += _oracle_time(lambda: attention(qb[:, :, h:h + 1], kb[:, :, h:h + 1],
                                                 vb[:, :, h:h + 1], causal=cfg.causal, scale=scale))
            n += 1
            if dt >= budget_s:
                break
        if dt >= budget_s:
            break
    fl = accounting.flops(1, n, cfg.S, cfg.D, cfg.causal)
    total = cfg.B * cfg.H
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "blas_threads": _host_threads(), "kind": "oracle",
            "sample": f"{n} of the {total} whole (batch, head) slices of {cfg.describe()} "
                      f"(every row against every key it sees), fp64 numpy, {dt:.1f} s",
            "extrapolated_full_workload_seconds": round(dt * total / n, 1)}


def calibration_copy(mib: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    if mib <= 0:
        return
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"  calibration copy: {mib} MiB x 3")


def side(args, synth):
    """One side figure on its own (used for its rocprofv3 summaries and tuning sweeps)."""
    name = args.side
    if name in synth.DECODE_CONFIGS:
        r = time_decode(synth.DECODE_CONFIGS[name], args.steps, args.warmup, args.settle_ms)
    elif name.endswith("_fp8"):
        r = time_fp8(synth.CONFIGS[name[:-4]], args.steps, args.warmup, args.settle_ms)
    elif name.endswith("_bwd"):
        r = time_backward(synth.CONFIGS[name[:-4]], args.steps, args.warmup, args.settle_ms)
    else:
        c = synth.CONFIGS[name]
        r2 = time_workload(c, args.steps, args.warmup, settle_ms=args.settle_ms,
                           tile_rows=args.tile_rows, key_split=args.key_split,
                           head_group=args.head_group)
        r = {"workload": c.describe(), "us_per_call": round(r2["ms"] * 1e3, 2),
             "tflops": round(r2["tflops"], 1), "frac_of_peak": round(r2["tflops"] / PEAK_TFLOPS, 4),
             "tile_rows": args.tile_rows, "key_split": args.key_split,
             "head_group": args.head_group,
             "settle": r2["settle"], "clock": r2["clock"]}
    log(f"  {name}: {r}")
    calibration_copy(args.calib_copy_mib)
    print(json.dumps({"side": name, "steps": args.steps, "warmup": args.warmup, **r}), flush=True)


def figure(r, peak=PEAK_TFLOPS):
    """Line entry of one forward workload's timing."""
    clk = r.get("clock") or {}
    mhz = clk.get("sclk_mhz")
    return {"us_per_call": round(r["ms"] * 1e3, 2), "tflops": round(r["tflops"], 1),
            "frac_of_peak": round(r["tflops"] / peak, 4),
            "per_launch_us": r.get("per_launch_us"), "settle": r.get("settle"), "clock": clk,
            "frac_of_peak_at_observed_clock": (round(r["tflops"] / peak_at(mhz), 4)
                                               if mhz else None)}


def main():
    global CLOCK
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed launches for about this long between warm-up and the timed loop")
    ap.add_argument("--workload", default="llama", help="key of synth.CONFIGS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the side figures (the other workloads, FP8, backward, decode)")
    ap.add_argument("--side", default=None,
                    help="time only this side figure (a key of synth.CONFIGS or synth.DECODE_CONFIGS) "
                         "and print it as one JSON line")
    ap.add_argument("--tile-rows", type=int, default=0, help="--side forward: 128 or 256 (0: auto)")
    ap.add_argument("--key-split", type=int, default=0, help="--side forward: 1 or 2 wave groups per tile (0: auto)")
    ap.add_argument("--head-group", type=int, default=0, help="--side forward: heads per XCD group (0: auto)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the (batch, head) split needs no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from scaled_dot_product_08_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.load_library()
    CLOCK = ClockSampler().start()
    if args.side is not None:
        side(args, synth)
        CLOCK.stop()
        return
    cfg = synth.CONFIGS[args.workload]
    log(f"workload {cfg.describe()}: warmup {args.warmup}, settle {args.settle_ms} ms, steps {args.steps}")
    r = time_workload(cfg, args.steps, args.warmup, samples=20, settle_ms=args.settle_ms)
    log(f"  {r['ms'] * 1e3:.1f} us/step, {r['tflops']:.1f} TFLOP/s; per launch {r['per_launch_us']}; "
        f"clock {r['clock']}")

    also = {}
    side_settle = min(args.settle_ms, 200.0)
    if not args.no_extra:
        for name in ("tiny", "mha", "mha_causal", "long", "varlen", "llama_alibi", "window128k"):
            c2 = synth.CONFIGS[name]
            # launch-bound small problems get more launches; the 64K-token ones fewer
            n = {"tiny": 1000, "long": 20, "varlen": 50}.get(name, max(100, args.steps))
            r2 = time_workload(c2, n, min(n, max(20, args.warmup)), samples=20,
                               settle_ms=side_settle)
            also[name] = {"workload": c2.describe(), **figure(r2)}
            log(f"  {name}: {r2['ms'] * 1e3:.1f} us, {r2['tflops']:.1f} TFLOP/s")

        r5 = time_fp8(synth.CONFIGS["llama"], max(100, args.steps), max(100, args.warmup), side_settle)
        also["llama_fp8"] = r5
        log(f"  llama_fp8: {r5['us_per_call']:.1f} us, {r5['tflops']:.1f} TFLOP/s")
        for name in ("llama", "mha"):
            r4 = time_backward(synth.CONFIGS[name], max(50, args.steps // 2), max(20, args.warmup // 5),
                               side_settle)
            also[name + "_bwd"] = r4
            log(f"  {name}_bwd: {r4['us_per_call']:.1f} us, {r4['tflops']:.1f} TFLOP/s")
        for name, c3 in synth.DECODE_CONFIGS.items():
            r3 = time_decode(c3, max(100, args.steps), max(50, args.warmup), side_settle)
            also[name] = r3
            log(f"  {name}: {r3['us_per_call']:.1f} us, {r3['GB_per_s']:.0f} GB/s "
                f"({100 * r3['frac_of_hbm_peak']:.1f} % of HBM peak)")
    CLOCK.stop()

    calibration_copy(args.calib_copy_mib)

    traffic = read_traffic(args.workload)
    clk = r["clock"] or {}
    mhz = clk.get("sclk_mhz")
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {**r["settle"], "note": "untimed launches between warm-up and the timed loop, enqueued back to back with it"},
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape; no weights)",
        "config": {"workload": cfg.describe(), "B": cfg.B, "H": cfg.H, "S": cfg.S, "D": cfg.D,
                   "causal": cfg.causal, "layout": "BSHD", "parallelism": "single GPU",
                   "input_sha256": r["sha256"][:16]},
        "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(r["tflops"] / PEAK_TFLOPS, 4),
                     "traffic": traffic, "algorithmic_bytes": r["bytes"],
                     "per_launch_us": r["per_launch_us"], "device_peak": device_peak(),
                     "observed_clock": clk, "peak_at_observed_clock": peak_at(mhz),
                     "frac_at_observed_clock": (round(r["tflops"] / peak_at(mhz), 4)
                                                if mhz else None),
                     "kernel_source": kernel_source_hash()},
        "also": also,
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        log("  timing the CPU oracle on the whole workload ...")
        line["cpu_baseline"] = cpu_baseline(cfg)
        if not args.no_extra:
            timings = {}
            for name in ("tiny", "mha", "mha_causal", "long", "varlen"):
                timings[name] = oracle_config_timing(name)
                log(f"  oracle {name}: {timings[name]}")
            line["cpu_baseline"]["per_workload"] = timings
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
