"""Attention-forward benchmark: TFLOP/s and fraction of MI355X dense MFMA peak.

One step = one call of the fused attention forward (the whole hot path: one
kernel launch) over one batch of synthetic input already resident in HBM.
Default workload: the LLaMA-2-7B-shaped layer, B=4 H=32 S=4096 D=128 bf16
causal (Q/K/V ~ N(0,1)*0.5). Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MFMA peak (B4 H12 S2048 D64 fp16; S4096 D128 bf16)"
PEAK_TFLOPS = 2516.6          # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E peak bandwidth
PEAK_TFLOPS_FP8 = 5033.2      # MI355X dense fp8 MFMA: twice the fp16/bf16 rate
KERNEL_SOURCES = ["scaled_dot_product_08_amd/csrc/attn_fwd_kernel.hip",
                  "scaled_dot_product_08_amd/csrc/attn_kernel.h"]
DECODE_SOURCES = ["scaled_dot_product_08_amd/csrc/attn_decode_kernel.hip",
                  "scaled_dot_product_08_amd/csrc/attn_decode.h"]


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in (sources or KERNEL_SOURCES):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_device_inputs(cfg):
    import numpy as np
    import torch

    import synth
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    inp = synth.make_inputs(cfg)
    dev = [torch.from_numpy(x.view(np.int16)).view(dt).cuda() for x in (inp.q, inp.k, inp.v)]
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).cuda()
    return inp, dev, cu


def time_workload(cfg, steps: int, warmup: int, samples: int = 0):
    """Mean over ``steps`` back-to-back launches bracketed by events; with ``samples``,
    also that many individually timed launches afterwards (median and minimum)."""
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
                         alibi_slopes=slopes)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    res = {"ms": ms, "flops": fl, "bytes": nbytes, "tflops": fl / (ms * 1e-3) / 1e12,
           "sha256": inp.sha256}
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


def time_fp8(cfg, steps: int, warmup: int):
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": cfg.describe().replace(cfg.dtype, "e4m3 (bf16 out)"),
            "us_per_call": round(ms * 1e3, 2), "tflops": round(tf, 1),
            "frac_of_fp8_peak": round(tf / PEAK_TFLOPS_FP8, 4)}


def time_backward(cfg, steps: int, warmup: int):
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": "backward " + cfg.describe(), "us_per_call": round(ms * 1e3, 2),
            "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS, 4)}


def time_decode(cfg, steps: int, warmup: int):
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    nbytes = accounting.decode_bytes(cfg.B, cfg.H, cfg.Sq, cfg.D, lens, cfg.dtype)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": cfg.describe(), "us_per_call": round(ms * 1e3, 2),
            "algorithmic_bytes": nbytes, "GB_per_s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "tflops": round(accounting.decode_flops(cfg.H, cfg.Sq, cfg.D, lens) / (ms * 1e-3) / 1e12, 2),
            "traffic": read_traffic(cfg.name, DECODE_SOURCES),
            "kernel_source": kernel_source_hash(DECODE_SOURCES)}


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


def cpu_baseline(cfg, budget_s: float = 12.0):
    """The fp64 oracle on a bounded sample of the same workload, timed on this host's cores."""
    import numpy as np

    import synth
    from oracle import attention_rows
    from scaled_dot_product_08_amd import accounting

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    inp = synth.make_inputs(cfg)
    scale = float(np.float32(1.0 / math.sqrt(cfg.D)))
    if cfg.varlen:
        # the longest packed sequence, all heads
        cu = inp.cu_seqlens
        s_best = int(np.argmax(np.diff(cu)))
        a, e = int(cu[s_best]), int(cu[s_best + 1])
        batches = [(inp.q[a:e], inp.k[a:e], inp.v[a:e])]
    else:
        batches = [(inp.q[b], inp.k[b], inp.v[b]) for b in range(cfg.B)]
    S = batches[0][0].shape[0]
    rows = np.arange(S)
    done = 0
    dt = 0.0
    for qb, kb, vb in batches:
        qf, kf, vf = (synth.bits_to_f64(x, cfg.dtype) for x in (qb, kb, vb))
        for h in range(cfg.H):
            t0 = time.perf_counter()
            attention_rows(qf, kf, vf, rows, causal=cfg.causal, scale=scale, heads=[h])
            dt += time.perf_counter() - t0
            done += 1
            if dt >= budget_s:
                break
        if dt >= budget_s:
            break
    fl = done * accounting.flops(1, 1, S, cfg.D, cfg.causal)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"{done} full (sequence, head) slices of S={S} rows (all keys each row sees), fp64 numpy, {dt:.1f} s"}


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
    """One side figure on its own (used for its rocprofv3 summaries)."""
    name = args.side
    if name in synth.DECODE_CONFIGS:
        r = time_decode(synth.DECODE_CONFIGS[name], args.steps, args.warmup)
    elif name.endswith("_fp8"):
        r = time_fp8(synth.CONFIGS[name[:-4]], args.steps, args.warmup)
    elif name.endswith("_bwd"):
        r = time_backward(synth.CONFIGS[name[:-4]], args.steps, args.warmup)
    else:
        c = synth.CONFIGS[name]
        r2 = time_workload(c, args.steps, args.warmup)
        r = {"workload": c.describe(), "us_per_call": round(r2["ms"] * 1e3, 2),
             "tflops": round(r2["tflops"], 1), "frac_of_peak": round(r2["tflops"] / PEAK_TFLOPS, 4)}
    log(f"  {name}: {r}")
    calibration_copy(args.calib_copy_mib)
    print(json.dumps({"side": name, "steps": args.steps, "warmup": args.warmup, **r}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="llama", help="key of synth.CONFIGS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the side figures (B4 H12 S2048 D64, ALiBi, 128K window)")
    ap.add_argument("--side", default=None,
                    help="time only this side figure (a key of synth.CONFIGS or synth.DECODE_CONFIGS) "
                         "and print it as one JSON line")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the (batch, head) split needs no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from scaled_dot_product_08_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.load_library()
    if args.side is not None:
        side(args, synth)
        return
    cfg = synth.CONFIGS[args.workload]
    log(f"workload {cfg.describe()}: warmup {args.warmup}, steps {args.steps}")
    r = time_workload(cfg, args.steps, args.warmup, samples=20)
    log(f"  {r['ms'] * 1e3:.1f} us/step, {r['tflops']:.1f} TFLOP/s; per launch {r['per_launch_us']}")

    also = {}
    if not args.no_extra:
        for name in ("tiny", "mha", "mha_causal", "long", "varlen", "llama_alibi", "window128k"):
            c2 = synth.CONFIGS[name]
            # launch-bound small problems get more launches; the 64K-token ones fewer
            n = {"tiny": 1000, "long": 20, "varlen": 50}.get(name, max(100, args.steps))
            r2 = time_workload(c2, n, min(n, max(20, args.warmup)), samples=20)
            also[name] = {"workload": c2.describe(), "us_per_call": round(r2["ms"] * 1e3, 2),
                          "tflops": round(r2["tflops"], 1),
                          "frac_of_peak": round(r2["tflops"] / PEAK_TFLOPS, 4),
                          "per_launch_us": r2["per_launch_us"]}
            log(f"  {name}: {r2['ms'] * 1e3:.1f} us, {r2['tflops']:.1f} TFLOP/s")

    if not args.no_extra:
        r5 = time_fp8(synth.CONFIGS["llama"], max(100, args.steps), max(100, args.warmup))
        also["llama_fp8"] = r5
        log(f"  llama_fp8: {r5['us_per_call']:.1f} us, {r5['tflops']:.1f} TFLOP/s")
        for name in ("llama", "mha"):
            r4 = time_backward(synth.CONFIGS[name], max(50, args.steps // 2), max(20, args.warmup // 5))
            also[name + "_bwd"] = r4
            log(f"  {name}_bwd: {r4['us_per_call']:.1f} us, {r4['tflops']:.1f} TFLOP/s")
        for name, c3 in synth.DECODE_CONFIGS.items():
            r3 = time_decode(c3, max(100, args.steps), max(50, args.warmup))
            also[name] = r3
            log(f"  {name}: {r3['us_per_call']:.1f} us, {r3['GB_per_s']:.0f} GB/s "
                f"({100 * r3['frac_of_hbm_peak']:.1f} % of HBM peak)")

    calibration_copy(args.calib_copy_mib)

    traffic = read_traffic(args.workload)
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
                     "kernel_source": kernel_source_hash()},
        "also": also,
    }
    if not args.no_cpu_baseline:
        log("  timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
