#!/usr/bin/env python3
"""Benchmark of the fused exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input, as a training step runs it: the fused forward that keeps O's
rounding residual for the backward (fa_fwd_train), then the backward's three
phases as fa_bwd_train runs them (per-head scale factors, D = rowsum(dO * O)
and fp16 tile images; dQ; dK/dV), on the causal bf16 workload B=4 H=16 N=4096
d=128 with upstream gradient dO. The line also gives the time of the same step
through fa_fwd and fa_bwd (no residual: the dQ pass then forms D itself). ``value`` is counted TFLOP/s of that step,
with the counted flops 4*B*H*N^2*d (halved for causal) for the forward and
2.5x that for the backward. Inputs are resident in HBM before timing starts.

Prints exactly one JSON line (on rank 0). Options:
  --gpus N        only N=1 is meaningful: this path runs on one GPU
  --steps K       timed steps (default 20)
  --warmup W      untimed warm-up steps (default 5)
  --no-sweep      skip the timing of the other workloads: the forward at head
                  sizes 64, 128 and 256, the backward at 256, the shared-K/V-head (grouped-query)
                  forward and backward, decoding, the chunked-prefill
                  (Nq != Nk) forward and backward, and the e4m3 (fp8) forward.
                  Each is timed warm and cold (CallTimer: median over >= 20
                  calls and >= 200 ms, the cold run with 512 MiB written
                  between calls)
  --no-cpu        skip the CPU oracle baseline
  --counters      instead: run two steps and a plain 512 MiB device copy and
                  exit (the program to run under rocprofv3 --pmc FETCH_SIZE,
                  then --pmc WRITE_SIZE)
  --write-traffic FETCH_DIR WRITE_DIR
                  instead: turn the two counter runs' CSV output into
                  profiles/traffic.json (HBM bytes per launch, scaled by what
                  the counters read for the copy of known size)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak at N=2k–16k, d=64/128"
# MI355X dense bf16 MFMA: 256 CUs x 4096 flop/clk x 2.4 GHz (AMD's 2.5 PFLOP/s).
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
HEADLINE = "bf16_b4h16n4096d128_causal_bwd"
SWEEP = ["bf16_b8h16n2048d64", "bf16_b8h16n2048d64_causal", "bf16_b2h32n8192d128_causal_x3",
         "bf16_b1h16n16384d128_causal", "bf16_b4h16n4096d128_causal_bwd"]
KERNEL_SOURCES = ["fa_device.hpp", "fa_kernels.hpp", "fa_api.hip", "fa_fwd.hip", "fa_fwd256.hip",
                  "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_decode.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 512 << 20          # the calibration copy reads and writes this much
# Kernel-name fragments -> the step's kernel names.
KERNEL_KEYS = {"fwd_bf16_kernel": "fwd", "bwd_dq_kernel": "bwd_dq", "bwd_dkdv_kernel": "bwd_dkdv",
               "bwd_dkdv16_kernel": "bwd_dkdv", "bwd_dq16_kernel": "bwd_dq",
               "bwd_absmax_kernel": "bwd_absmax", "bwd_scale_kernel": "bwd_scale",
               "bwd_image_kernel": "bwd_image"}


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_41_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


WARMUP_CALLS = 5
MIN_CALLS = 20
MIN_TIMED_MS = 200.0
FLUSH_BYTES = 512 << 20         # written between calls for the cold (L2/MALL-flushed) time


PROBE_SAMPLES = 4000            # one every ~8128 shader clocks: ~15-25 ms of samples


def measure_sclk(fn, dev, min_ms: float = 50.0):
    """Shader clock (MHz) while ``fn`` runs back to back: fa_clock_probe's wave
    samples the shader-clock and 100 MHz counters on a second stream (default
    priority) while the calls run on the current one. The calls go on for at
    least min_ms, longer than the probe's samples take, and the middle 80% of
    the samples give the clock. None if the counters did not advance."""
    import torch

    import exact_attention_41_amd as fa
    samples = torch.zeros((PROBE_SAMPLES, 2), dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(device=dev)
    fn()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize(dev)
    est_ms = max((time.perf_counter() - t0) * 1e3, 1e-3)
    calls = max(1, int(min_ms / est_ms) + 1)
    fa.fa_clock_probe(samples, sleep_units=1, stream=side)
    for _ in range(calls):
        fn()
    torch.cuda.synchronize(dev)
    x = samples.cpu().numpy()
    a, b = int(0.1 * len(x)), int(0.9 * len(x)) - 1
    dt, dr = int(x[b, 0] - x[a, 0]), int(x[b, 1] - x[a, 1])
    if dt <= 0 or dr <= 0:
        return None
    return round(dt / dr * 100.0, 1)


class CallTimer:
    """Median device time of one call: WARMUP_CALLS untimed calls, then at
    least MIN_CALLS timed ones covering at least MIN_TIMED_MS in total, each
    bracketed by events on the current stream. ``cold`` writes FLUSH_BYTES
    before every timed call (outside its events), so the call starts with the
    2nd-level caches and the last-level cache holding nothing of its inputs."""

    def __init__(self, dev):
        import torch
        self.torch = torch
        self.dev = dev
        self.flush_buf = None

    def _calls(self, fn, n, flush):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i in range(n):
            if flush:
                self.flush_buf.fill_(i & 0xFF)
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize(self.dev)
        return [a.elapsed_time(b) for a, b in ev]

    def median(self, fn, cold: bool = False):
        torch = self.torch
        if cold and self.flush_buf is None:
            self.flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=self.dev)
        for _ in range(WARMUP_CALLS):
            fn()
        probe = self._calls(fn, 3, cold)
        est = max(sorted(probe)[1], 1e-3)
        n = min(max(MIN_CALLS, int(MIN_TIMED_MS / est) + 1), 5000)
        times = sorted(self._calls(fn, n, cold))
        return times[len(times) // 2], n

    def both(self, fn):
        """(warm median ms, cold median ms, timed calls of the warm run)."""
        warm, n = self.median(fn)
        cold, _ = self.median(fn, cold=True)
        return warm, cold, n


# ---------------------------------------------------------------------------
def gpu_step_timing(w, steps: int, warmup: int, with_clock: bool = True):
    import torch

    import exact_attention_41_amd as fa
    from exact_attention_41_amd import workloads as wl

    dev = torch.device("cuda:0")
    inp = wl.workload_inputs(w)
    q, k, v, do = (wl.to_device(x, "bf16", dev) for x in (inp.q, inp.k, inp.v, inp.do))
    o, o_res = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    names = ["fwd", "bwd_preprocess", "bwd_dq", "bwd_dkdv"]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, o_res=o_res)
        if ev is not None:
            ev[1].record()
        fa.fa_bwd_preprocess(q, k, v, o, do, ws, o_res=o_res)
        if ev is not None:
            ev[2].record()
        fa.fa_bwd_dq(q, k, v, do, lse, ws, dq, causal=w.causal, scale=w.scale, d_ready=True)
        if ev is not None:
            ev[3].record()
        fa.fa_bwd_dkdv(q, k, v, do, ws, dk, dv, causal=w.causal, scale=w.scale)
        if ev is not None:
            ev[4].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for s in range(steps):
        step(events[s])
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    per_kernel = {n: 0.0 for n in names}
    for ev in events:
        for i, n in enumerate(names):
            per_kernel[n] += ev[i].elapsed_time(ev[i + 1])
    per_kernel = {n: t / steps for n, t in per_kernel.items()}
    ms_per_step = (t1 - t0) * 1000.0 / steps
    # The shader clock while the whole step runs, and while each kernel runs
    # on its own (back to back; the workspace holds what the later phases
    # read).
    kernels = {
        "fwd": lambda: fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse,
                                 o_res=o_res),
        "bwd_preprocess": lambda: fa.fa_bwd_preprocess(q, k, v, o, do, ws, o_res=o_res),
        "bwd_dq": lambda: fa.fa_bwd_dq(q, k, v, do, lse, ws, dq, causal=w.causal,
                                       scale=w.scale, d_ready=True),
        "bwd_dkdv": lambda: fa.fa_bwd_dkdv(q, k, v, do, ws, dk, dv, causal=w.causal,
                                           scale=w.scale),
    }
    clocks = {}
    if with_clock:
        clocks["step"] = measure_sclk(step, dev)
        for n in names:
            clocks[n] = measure_sclk(kernels[n], dev)
    log("bench: shader clock (MHz) " + ", ".join(f"{k}={v}" for k, v in clocks.items()))
    if with_clock:
        # For comparison (not part of the step): the preprocess and dQ pass of
        # a backward given no residual, where the dQ pass forms D itself.
        timer = CallTimer(dev)
        per_kernel["bwd_preprocess_no_res"] = timer.median(
            lambda: fa.fa_bwd_preprocess(q, k, v, o, do, ws))[0]
        per_kernel["bwd_dq_no_res"] = timer.median(
            lambda: fa.fa_bwd_dq(q, k, v, do, lse, ws, dq, causal=w.causal, scale=w.scale,
                                 d_ready=False))[0]

        def plain_step():
            fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
            fa.fa_bwd(q, k, v, o, do, lse, causal=w.causal, scale=w.scale, dq=dq, dk=dk,
                      dv=dv, workspace=ws)
        per_kernel["step_fa_fwd_fa_bwd"] = timer.median(plain_step)[0]
    return ms_per_step, per_kernel, clocks


def gpu_forward_sweep(names):
    """bf16 forward of each workload: warm and cold medians (CallTimer), and
    the device memory one call takes beyond its inputs and outputs (free
    memory before and after the call, and torch's allocation peak): the
    forward keeps no N x N buffer, so both are expected to be 0."""
    import torch

    import exact_attention_41_amd as fa
    from exact_attention_41_amd import workloads as wl

    out = []
    dev = torch.device("cuda:0")
    timer = CallTimer(dev)
    for name in names:
        w = wl.WORKLOADS[name] if name in wl.WORKLOADS else wl.WIDE_WORKLOADS[name]
        inp = wl.make_inputs(w.B, w.H, w.N, w.d, "bf16", w.seed, w.qk_mult)
        q, k, v = (wl.to_device(x, "bf16", dev) for x in (inp.q, inp.k, inp.v))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def call():
            fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

        med, cold, n = timer.both(call)
        sclk = measure_sclk(call, dev)
        torch.cuda.synchronize(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        alloc0 = torch.cuda.memory_allocated(dev)
        free0 = torch.cuda.mem_get_info(dev)[0]
        call()
        torch.cuda.synchronize(dev)
        free1 = torch.cuda.mem_get_info(dev)[0]
        extra = {"free_bytes_delta": int(free0 - free1),
                 "torch_peak_delta": int(torch.cuda.max_memory_allocated(dev) - alloc0)}
        tf = w.fwd_flops() / (med * 1e-3) / 1e12
        ctf = w.fwd_flops() / (cold * 1e-3) / 1e12
        out.append({"workload": name, "pass": "fwd", "ms": round(med, 4),
                    "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                    "cold_ms": round(cold, 4), "cold_tflops": round(ctf, 1), "calls": n,
                    "sclk_mhz": sclk,
                    "frac_at_sclk": (round(tf / (256 * 4096 * sclk * 1e-6), 4) if sclk else None),
                    "extra_device_memory": extra})
        log(f"  fwd {name}: {med:.3f} ms  {tf:.1f} TFLOP/s  {100 * tf / PEAK_BF16_TFLOPS:.1f}%  "
            f"(cold {cold:.3f} ms; shader clock {sclk} MHz; extra memory {extra})")
        del q, k, v, o, lse
    return out


def counter_pass(w) -> int:
    """Two steps of the path, then a plain copy of COPY_BYTES (torch.neg, one
    read and one write per element) whose counter readings calibrate the
    HBM byte counts."""
    import torch

    ms, _, _ = gpu_step_timing(w, steps=2, warmup=1, with_clock=False)
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"bench --counters: 2 steps ({ms:.3f} ms/step) and 2 copies of {COPY_BYTES >> 20} MiB done")
    return 0


def _counter_means(run_dir: str, counter: str):
    """Mean per dispatch of one derived counter, by kernel key (and the copy)."""
    import csv
    import glob

    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per_dispatch = {}
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = next((v for k, v in KERNEL_KEYS.items() if k in name), None)
            if key is None and "neg" in name:
                key = "copy"
            if key is None:
                continue
            d = per_dispatch.setdefault(key, {})
            d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per_dispatch.items()}


def write_traffic(fetch_dir: str, write_dir: str) -> int:
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    known_kib = COPY_BYTES / 1024.0
    fs, ws = known_kib / fetch["copy"], known_kib / write["copy"]
    kernels = {}
    for key in sorted(set(fetch) & set(write) - {"copy"}):
        kernels[key] = {"fetch_kib": round(fetch[key], 1), "write_kib": round(write[key], 1),
                        "hbm_bytes_per_launch": int(round((fetch[key] * fs + write[key] * ws) * 1024))}
    out = {"source_sha": kernel_source_sha(), "workload": HEADLINE,
           "copy_probe": {"bytes_each_way": COPY_BYTES, "fetch_kib": round(fetch["copy"], 1),
                          "write_kib": round(write["copy"], 1), "fetch_scale": round(fs, 4),
                          "write_scale": round(ws, 4)},
           "kernels": kernels}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    log(f"wrote {TRAFFIC_FILE}")
    return 0


def gpu_gqa_timing(names):
    """Forward and backward of the shared-K/V-head workloads (fa_fwd_gqa,
    fa_bwd_gqa), warm and cold medians (CallTimer); flops counted as for the
    other workloads (over the H query heads)."""
    import torch

    import exact_attention_41_amd as fa
    from exact_attention_41_amd import workloads as wl

    out = []
    dev = torch.device("cuda:0")
    timer = CallTimer(dev)
    for name in names:
        w = wl.GQA_WORKLOADS[name]
        inp = wl.workload_inputs(w)
        q, k, v, do = (wl.to_device(x, "bf16", dev) for x in (inp.q, inp.k, inp.v, inp.do))
        o, o_res = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_gqa_workspace_size(w.B, w.H, w.kv_heads, w.N, w.d),
                         dtype=torch.uint8, device=dev)

        def fwd():
            fa.fa_fwd_gqa(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, o_res=o_res)

        def bwd():
            fa.fa_bwd_gqa(q, k, v, o, do, lse, causal=w.causal, scale=w.scale, dq=dq, dk=dk,
                          dv=dv, workspace=ws, o_res=o_res)

        res = {label: timer.both(fn) for label, fn in (("fwd", fwd), ("bwd", bwd))}
        ftf = w.fwd_flops() / (res["fwd"][0] * 1e-3) / 1e12
        btf = w.bwd_flops() / (res["bwd"][0] * 1e-3) / 1e12
        out.append({"workload": name, "H": w.H, "Hkv": w.kv_heads,
                    "fwd_ms": round(res["fwd"][0], 4), "fwd_tflops": round(ftf, 1),
                    "fwd_frac_peak": round(ftf / PEAK_BF16_TFLOPS, 4),
                    "fwd_cold_ms": round(res["fwd"][1], 4),
                    "bwd_ms": round(res["bwd"][0], 4), "bwd_tflops": round(btf, 1),
                    "bwd_frac_peak": round(btf / PEAK_BF16_TFLOPS, 4),
                    "bwd_cold_ms": round(res["bwd"][1], 4)})
        log(f"  gqa {name}: fwd {res['fwd'][0]:.3f} ms {ftf:.1f} TFLOP/s, "
            f"bwd {res['bwd'][0]:.3f} ms {btf:.1f} TFLOP/s (cold {res['fwd'][1]:.3f}, "
            f"{res['bwd'][1]:.3f} ms)")
        del q, k, v, do, o, o_res, lse, dq, dk, dv, ws
    return out


def gpu_wide_bwd_timing(names):
    """Backward at head size 256 (fa_bwd, d = 256), warm and cold medians;
    flops counted as 2.5x the forward's."""
    import torch

    import exact_attention_41_amd as fa
    from exact_attention_41_amd import workloads as wl

    out = []
    dev = torch.device("cuda:0")
    timer = CallTimer(dev)
    for name in names:
        w = wl.WIDE_WORKLOADS[name]
        inp = wl.make_inputs(w.B, w.H, w.N, w.d, "bf16", w.seed, with_do=True)
        q, k, v, do = (wl.to_device(x, "bf16", dev) for x in (inp.q, inp.k, inp.v, inp.do))
        o, o_res = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, o_res=o_res)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8,
                         device=dev)

        def call():
            fa.fa_bwd(q, k, v, o, do, lse, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                      workspace=ws, o_res=o_res)

        med, cold, n = timer.both(call)
        tf = w.bwd_flops() / (med * 1e-3) / 1e12
        out.append({"workload": name, "pass": "bwd", "ms": round(med, 4), "tflops": round(tf, 1),
                    "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "cold_ms": round(cold, 4),
                    "calls": n})
        log(f"  bwd {name}: {med:.3f} ms  {tf:.1f} TFLOP/s  {100 * tf / PEAK_BF16_TFLOPS:.1f}% "
            f"(cold {cold:.3f} ms)")
        del q, k, v, do, o, o_res, lse, dq, dk, dv, ws
    return out


def gpu_rect_timing(names):
    """Forward and backward with Nq query rows against Nk keys (fa_fwd_rect,
    fa_bwd_rect), warm and cold medians (CallTimer); flops counted over the
    unmasked score elements (the backward as 2.5x the forward)."""
    import torch

    import exact_attention_41_amd as fa
    from exact_attention_41_amd import workloads as wl

    out = []
    dev = torch.device("cuda:0")
    timer = CallTimer(dev)
    for name in names:
        w = wl.RECT_WORKLOADS[name]
        inp = wl.make_decode_inputs(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed, with_do=True)
        q, k, v, do = (wl.to_device(x, "bf16", dev) for x in (inp.q, inp.k, inp.v, inp.do))
        o, o_res = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_rect_workspace_size(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d),
                         dtype=torch.uint8, device=dev)

        def fwd():
            fa.fa_fwd_rect(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, o_res=o_res)

        def bwd():
            fa.fa_bwd_rect(q, k, v, o, do, lse, causal=w.causal, scale=w.scale, dq=dq, dk=dk,
                           dv=dv, workspace=ws, o_res=o_res)

        res = {label: timer.both(fn) for label, fn in (("fwd", fwd), ("bwd", bwd))}
        ftf = wl.rect_flops(w) / (res["fwd"][0] * 1e-3) / 1e12
        btf = 2.5 * wl.rect_flops(w) / (res["bwd"][0] * 1e-3) / 1e12
        out.append({"workload": name, "Nq": w.Nq, "Nk": w.Nk, "H": w.H, "Hkv": w.Hkv,
                    "ms": round(res["fwd"][0], 4), "tflops": round(ftf, 1),
                    "frac_peak": round(ftf / PEAK_BF16_TFLOPS, 4),
                    "cold_ms": round(res["fwd"][1], 4),
                    "bwd_ms": round(res["bwd"][0], 4), "bwd_tflops": round(btf, 1),
                    "bwd_frac_peak": round(btf / PEAK_BF16_TFLOPS, 4),
                    "bwd_cold_ms": round(res["bwd"][1], 4)})
        log(f"  rect {name}: fwd {res['fwd'][0]:.3f} ms {ftf:.1f} TFLOP/s "
            f"{100 * ftf / PEAK_BF16_TFLOPS:.1f}%, bwd {res['bwd'][0]:.3f} ms {btf:.1f} TFLOP/s "
            f"{100 * btf / PEAK_BF16_TFLOPS:.1f}%")
        del q, k, v, do, o, o_res, lse, dq, dk, dv, ws
    return out


PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS    # dense e4m3 MFMA (AMD's 5.0 PFLOP/s)


def gpu_fp8_timing(names):
    """Forward with e4m3 operands (fa_fwd_fp8), warm and cold medians;
    flops counted as for the bf16 forward, against the fp8 MFMA peak."""
    import torch

    import exact_attention_41_amd as fa
    from exact_attention_41_amd import workloads as wl

    out = []
    dev = torch.device("cuda:0")
    timer = CallTimer(dev)
    for name in names:
        w = wl.FP8_WORKLOADS[name]
        inp = wl.make_fp8_inputs(w.B, w.H, w.H, w.N, w.N, w.d, w.seed)
        q, k, v = (wl.fp8_to_device(x, dev) for x in (inp.q8, inp.k8, inp.v8))
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def call():
            fa.fa_fwd_fp8(q, k, v, inp.dq, inp.dk, inp.dv, causal=w.causal, scale=w.scale,
                          out=o, lse=lse)

        med, cold, n = timer.both(call)
        tf = w.fwd_flops() / (med * 1e-3) / 1e12
        out.append({"workload": name, "pass": "fwd", "dtype": "e4m3", "ms": round(med, 4),
                    "tflops": round(tf, 1), "peak": round(PEAK_FP8_TFLOPS, 1),
                    "frac_peak": round(tf / PEAK_FP8_TFLOPS, 4), "cold_ms": round(cold, 4),
                    "calls": n})
        log(f"  fp8 {name}: {med:.3f} ms  {tf:.1f} TFLOP/s  {100 * tf / PEAK_FP8_TFLOPS:.1f}% "
            "of the fp8 peak")
        del q, k, v, o, lse
    return out


HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s


def gpu_decode_timing(names):
    """Split-K/V decoding (fa_decode): median time per call (warm; cold as
    well) and the rate at
    which it moves its algorithmic bytes (K and V once, q, O, lse), against
    the HBM roof."""
    import torch

    import exact_attention_41_amd as fa
    from exact_attention_41_amd import workloads as wl

    out = []
    dev = torch.device("cuda:0")
    timer = CallTimer(dev)
    for name in names:
        w = wl.DECODE_WORKLOADS[name]
        inp = wl.make_decode_inputs(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed)
        q, k, v = (wl.to_device(x, "bf16", dev) for x in (inp.q, inp.k, inp.v))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_decode_workspace_size(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d),
                         dtype=torch.uint8, device=dev)
        def call():
            fa.fa_decode(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)

        med, cold, n = timer.both(call)
        gbs = w.io_bytes() / (med * 1e-3) / 1e9
        out.append({"workload": name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk,
                    "d": w.d, "ms": round(med, 4), "bytes": w.io_bytes(),
                    "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(gbs / HBM_PEAK_GBS, 4)},
                    "cold_ms": round(cold, 4), "calls": n})
        log(f"  decode {name}: {med * 1000:.1f} us  {gbs:.0f} GB/s  "
            f"{100 * gbs / HBM_PEAK_GBS:.1f}% of HBM")
        del q, k, v, o, lse, ws
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def environment() -> dict:
    """Versions and hardware the numbers were taken with."""
    import numpy
    import torch
    props = torch.cuda.get_device_properties(0)
    return {"numpy": numpy.__version__, "torch": torch.__version__, "hip": torch.version.hip,
            "gpu": props.gcnArchName, "compute_units": props.multi_processor_count,
            "cpu_model": cpu_model()}


# ---------------------------------------------------------------------------
def cpu_baseline(w, min_seconds: float = 10.0):
    """The fp64 oracle, as it stands, on the host cores: fwd + bwd per head."""
    import concurrent.futures as cf

    import numpy as np

    from exact_attention_41_amd import workloads as wl
    from oracle import attention as ora

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    # The host's cores available to this process, and the threads used: at
    # most 16, one GPU's share of a host whose other GPUs may be busy.
    host_cores = len(os.sched_getaffinity(0))
    cores = min(host_cores, 16)
    inp = wl.workload_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        q, k, v, do = (x[b, h].astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))
        ora.head_fwd(q, k, v, w.causal, w.scale)
        ora.head_bwd(q, k, v, do, w.causal, w.scale)

    done = 0
    ctx = threadpool_limits(1) if threadpool_limits else None
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        while done < len(heads):
            batch = heads[done:done + cores]
            list(ex.map(one, batch))
            done += len(batch)
            if time.perf_counter() - t0 >= min_seconds:
                break
    elapsed = time.perf_counter() - t0
    if ctx is not None:
        ctx.unregister()
    per_head = (w.fwd_flops() + w.bwd_flops()) / len(heads)
    tflops = per_head * done / elapsed / 1e12
    return {"value": round(tflops, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "host_cores": host_cores, "host_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"{done} of {len(heads)} heads of {w.name} (fwd+bwd, fp64 numpy, "
                      f"S/P materialised), {elapsed:.1f} s wall; counted flops as on the GPU"}


# ---------------------------------------------------------------------------
def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--counters", action="store_true")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.write_traffic:
        return write_traffic(*args.write_traffic)
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this attention path is measured "
              "on one GPU only (heads shard across GPUs with no communication; see the design "
              "notes). Run with --gpus 1.", file=sys.stderr, flush=True)
        return 2
    rank = int(os.environ.get("RANK", "0"))

    import torch

    from exact_attention_41_amd import _lib
    from exact_attention_41_amd import workloads as wl

    _lib.load()   # raises if libfa.so was not built: there is no fallback
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    w = wl.WORKLOADS[HEADLINE]
    if args.counters:
        return counter_pass(w)
    log(f"bench: workload {w.name} steps={args.steps} warmup={args.warmup}")
    ms, per_kernel, clocks = gpu_step_timing(w, args.steps, args.warmup)
    plain_ms = per_kernel.pop("step_fa_fwd_fa_bwd", None)
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    value = (fwd_f + bwd_f) / (ms * 1e-3) / 1e12
    log(f"bench: {ms:.3f} ms/step, {value:.1f} TFLOP/s; per kernel (ms): "
        + ", ".join(f"{k}={v:.3f}" for k, v in per_kernel.items()))

    # Algorithmic MFMA flops each kernel performs over the unmasked score
    # elements (counted convention N^2/2 when causal): 4d per score forward
    # (Q K^T, P V), 6d for dQ (S, dP, dS K: D comes from the preprocess), 8d
    # for dK/dV (S, dP, dV, dK).
    alg = {"fwd": fwd_f, "bwd_dq": 1.5 * fwd_f, "bwd_dkdv": 2.0 * fwd_f}
    dominant = max(alg, key=lambda n: per_kernel[n])
    achieved = alg[dominant] / (per_kernel[dominant] * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            t = json.load(open(TRAFFIC_FILE))
            if t.get("source_sha") == kernel_source_sha() and dominant in t.get("kernels", {}):
                traffic = t["kernels"][dominant]["hbm_bytes_per_launch"]
        except (ValueError, KeyError, TypeError):
            traffic = None
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 1),
                "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    sclk = clocks.get(dominant)
    if sclk:
        # the same peak at the shader clock measured while the kernel ran
        peak_at = 256 * 4096 * sclk * 1e6 / 1e12
        roofline["sclk_mhz"] = sclk
        roofline["peak_at_sclk"] = round(peak_at, 1)
        roofline["frac_at_sclk"] = round(achieved / peak_at, 4)

    fwd_tf = fwd_f / (per_kernel["fwd"] * 1e-3) / 1e12
    bwd_ms = per_kernel["bwd_preprocess"] + per_kernel["bwd_dkdv"] + per_kernel["bwd_dq"]
    bwd_tf = bwd_f / (bwd_ms * 1e-3) / 1e12
    sweep = [] if args.no_sweep else gpu_forward_sweep(SWEEP)
    wide = [] if args.no_sweep else gpu_forward_sweep(list(wl.WIDE_WORKLOADS))
    wide_bwd = [] if args.no_sweep else gpu_wide_bwd_timing(list(wl.WIDE_WORKLOADS))
    gqa = [] if args.no_sweep else gpu_gqa_timing(list(wl.GQA_WORKLOADS))
    decode = [] if args.no_sweep else gpu_decode_timing(list(wl.DECODE_WORKLOADS))
    rect = [] if args.no_sweep else gpu_rect_timing(list(wl.RECT_WORKLOADS))
    fp8 = [] if args.no_sweep else gpu_fp8_timing(list(wl.FP8_WORKLOADS))
    cpu = None
    if not args.no_cpu and rank == 0:
        log("bench: timing the fp64 oracle on host cores")
        cpu = cpu_baseline(w)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v, dO; PCG64 seed 5; bf16 RNE)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "pass": "fwd+bwd", "parallelism": "single GPU"},
        "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"ms": round(per_kernel["fwd"], 4), "tflops": round(fwd_tf, 1),
                "frac_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_tf, 1),
                "frac_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4)},
        "kernel_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        # the same step through fa_fwd and fa_bwd (no residual kept), median
        # of single steps
        "step_fa_fwd_fa_bwd": None if plain_ms is None else {
            "ms": round(plain_ms, 4),
            "tflops": round((fwd_f + bwd_f) / (plain_ms * 1e-3) / 1e12, 2)},
        "sclk_mhz": clocks,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "forward_workloads": sweep,
        "wide_workloads": wide,
        "wide_bwd_workloads": wide_bwd,
        "gqa_workloads": gqa,
        "decode_workloads": decode,
        "rect_workloads": rect,
        "fp8_workloads": fp8,
        "kernel_source_sha": kernel_source_sha(),
        "timing": {"warmup_calls": WARMUP_CALLS, "min_calls": MIN_CALLS,
                   "min_timed_ms": MIN_TIMED_MS, "statistic": "median",
                   "cold": f"{FLUSH_BYTES >> 20} MiB written before each call"},
        "environment": environment(),
    }
    if rank == 0:
        print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
