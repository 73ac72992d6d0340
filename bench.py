"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole path over resident synthetic inputs:
  * prefill: fa_fwd on causal self-attention, B=1, H=32, L=16384, d=128, bf16
    (the pages' 16,384-token example), counted as 4*B*H*L*L*d/2 FLOP;
  * decode:  fa_decode (split-K + combine) on B=64 requests, 32 query / 8 KV heads,
    d=128, bf16 cache with per-request context lengths uniform in [8192, 32768],
    counted as the K and V bytes of every request's context.
The headline ``value`` is the prefill TFLOP/s from the median launch time; decode KV GB/s is
reported beside it, and the backward of the same prefill (fa_bwd, timed on its own after the
step) beside that. ``workloads`` then times each of the five workloads alone (K launches after
W warm-ups: the single-head fp32 check in microseconds only, the prefills in TFLOP/s and as a
fraction of the bf16 MFMA peak, decode in KV GB/s), and the FP8 prefill (fa_fwd_fp8) of the
16,384-token workload against the fp8 MFMA peak, launched in turn with the bf16 prefill of the
same workload for its speed-up. Kernel durations come from HIP events on the stream the kernels
run on (torch's current stream), over exactly K timed steps after W warm-up steps. Before its
warm-ups every timed section runs its calls untimed until their times have stopped falling
(at least SETTLE_MS of wall time, at most SETTLE_MAX_MS), so that the GPU has left the low
clock it starts from after being idle or after a lighter load; ``settle`` reports what each
section took.

``cpu_baseline`` times the CPU fp64 oracle (as it is, untuned) on a bounded sample of
the same prefill workload: consecutive blocks of query rows of one head, until about
ten seconds of CPU work, reported in the same unit (algorithmic TFLOP/s of the rows
it finished).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bf16 attn-fwd TFLOP/s & % MFMA peak at L=16k d=128; decode KV-read GB/s"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
# The pages' own figure, quoted as context only: another vendor's part, not a target.
CONTEXT = {"fa2_forward_flops_utilisation_a100": "50-70% of theoretical peak",
           "hardware": "NVIDIA A100 (another vendor's part)",
           "source": "'2.1 FlashAttention-2 的核心思想' §2.1.6 and §2.1.10 (quoting the official report)",
           "use": "context only; not comparable to an MI355X fraction and not a target"}
# Backward work counted as five products of the forward's size (S, dP, dV, dK, dQ):
# 2.5 times the forward's FLOP, whatever the kernels recompute.
BWD_FLOP_PER_FWD = 2.5
PREFILL = "causal_prefill_B1_H32_L16384_d128"
DECODE = "decode_B64_H32_Hkv8_ctx32768_d128"
# Sources whose compiled kernels a committed counter profile describes.
KERNEL_SOURCES = {"prefill": ["fa_fwd.hip", "fa_tiles.h", "fa_device.h", "fa_launch.h"],
                  "fp8": ["fa_fwd_fp8.hip", "fa_tiles.h", "fa_device.h", "fa_launch.h"],
                  "decode": ["fa_decode.hip", "fa_device.h", "fa_launch.h"],
                  "backward": ["fa_bwd.hip", "fa_tiles.h", "fa_device.h", "fa_launch.h"]}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--window", type=int, default=None,
                    help="with --only: a sliding window of this many keys (prefill, backward and decode workloads); "
                         "work is counted over the keys inside the window")
    ap.add_argument("--fp8", action="store_true",
                    help="with --only and a prefill workload (d = 128): FP8 E4M3 inputs through fa_fwd_fp8")
    ap.add_argument("--page", type=int, default=None,
                    help="with --only and a decode workload: the KV cache in pages of this many positions, "
                         "scattered through a pool by a random block table (fa_decode_paged)")
    ap.add_argument("--only", default=None,
                    help="time one part alone (for profiling): prefill, decode, backward, copy, any workload name of "
                         "fa_inputs.WORKLOADS, or backward:<prefill workload>; prints a short JSON line "
                         "instead of the bench line")
    return ap.parse_args()


def source_digest(part):
    """First 16 hex digits of sha256 over the kernel sources of one part, in order."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[part]:
        with open(os.path.join(ROOT, "exact_attention_111_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(part, workload=None):
    """Calibrated HBM bytes per launch of one part (and workload, if given; records without a
    workload are the part's bench workload), from the `traffic-record:` line of a rocprofv3
    FETCH_SIZE/WRITE_SIZE summary under profiles/. Returned only while the kernel sources
    are byte-identical to the ones profiled; otherwise (None, reason)."""
    want = source_digest(part)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path, encoding="utf-8") as fh:
            for line in fh:
                if not line.startswith("traffic-record:"):
                    continue
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("part") != part or rec.get("workload") != workload:
                    continue
                if rec.get("source_sha256_16") != want:
                    return None, f"{os.path.relpath(path, ROOT)} profiled other sources"
                return rec, os.path.relpath(path, ROOT)
    return None, "no counter profile"


def host_cpu():
    """The host CPU model and its logical core count (for the CPU baseline)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return model, os.cpu_count()


def cpu_baseline(w, x, seconds):
    """Time the fp64 oracle on 256-row blocks of query rows, newest rows first, head after
    head, until about `seconds` of CPU work; report algorithmic TFLOP/s of those rows."""
    import numpy as np

    import fa_inputs
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    block = 256
    flops = 0.0
    rows_done = 0
    heads_touched = 0
    t0 = time.perf_counter()
    for h in range(w.H):
        if time.perf_counter() - t0 >= seconds:
            break
        q = fa_inputs.as_oracle_f64(x["q"][0, h])
        k = fa_inputs.as_oracle_f64(x["k"][0, h * w.Hkv // w.H])
        v = fa_inputs.as_oracle_f64(x["v"][0, h * w.Hkv // w.H])
        heads_touched += 1
        L, d = q.shape
        hi = L
        while hi > 0 and time.perf_counter() - t0 < seconds:
            rows = np.arange(max(0, hi - block), hi)
            oracle.attention_head(q, k, v, scale=w.scale, causal=True, rows=rows)
            flops += 4.0 * d * float((rows + 1).sum())  # visible (query, key) pairs of these rows
            rows_done += len(rows)
            hi -= block
    dt = time.perf_counter() - t0
    model, ncpu = host_cpu()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "host_cpu": model, "os_cpu_count": ncpu,
            "sample": f"{rows_done} query rows over {heads_touched} head(s) of {w.name} (newest rows first), "
                      f"fp64, {dt:.1f} s",
            "seconds": round(dt, 2)}


def spread(ms):
    """Median and 10th / 90th percentiles of per-launch times (ms)."""
    import statistics
    t = sorted(ms)
    pick = lambda f: t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]  # noqa: E731  (nearest rank)
    return {"ms_median": round(statistics.median(t), 4), "ms_p10": round(pick(0.1), 4), "ms_p90": round(pick(0.9), 4)}


def library_gemm_tflops(dev, n=16384, reps=10):
    """Context for the matrix-core roofline: a plain bf16 GEMM (n x n x n) through the vendor
    BLAS behind torch.matmul, on the same GPU in the same run; median of `reps` launches.
    It shows what a dense bf16 product reaches at the clock this GPU holds under load."""
    import torch
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    settle([lambda: torch.matmul(a, b, out=c)], "library_gemm")
    for _ in range(3):
        torch.matmul(a, b, out=c)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    ms = ts[len(ts) // 2]
    del a, b, c
    return {"tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4),
            "what": f"torch.matmul bf16 {n}x{n}x{n}, median of {reps}"}


def _window_pairs(lens, W):
    """Visible (query, key) pairs of causal self-attention with a window of W keys per query,
    summed over sequences of the given lengths: sum over i < n of min(W, i + 1)."""
    tot = 0
    for n in lens:
        n = int(n)
        m = min(n, W)
        tot += m * (m + 1) // 2 + (n - m) * W
    return float(tot)


def workload_call(w, dev, window=None, page=None, fp8=False):
    """One launch of a named workload on resident inputs, as a callable, with its algorithmic
    work per launch: (fn, work, unit). Prefill work is 4 H d per visible (query, key) pair,
    causal counted as half the square (TFLOP/s); decode work is the K and V bytes of every
    request's context (GB/s)."""
    import torch

    import exact_attention_111_amd as fa
    import fa_inputs
    if w.kind == "decode" and page is not None:
        x = fa_inputs.paged_decode_inputs(w.B, w.H, w.Hkv, w.L, w.d, page, seed=w.seed, device=dev,
                                          len_range=w.len_range)
    elif w.kind == "prefill" and fp8:
        x = fa_inputs.fp8_prefill_inputs(w.B, w.H, w.Hkv, w.L, w.L, w.d, seed=w.seed, device=dev,
                                         len_range=w.len_range)
    else:
        x = fa_inputs.workload_inputs(w, device=dev)
    if w.kind == "decode" and page is not None:
        o = torch.empty_like(x["q"])
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        cap = x["block_table"].shape[1] * page
        ws = torch.empty(max(16, fa.decode_workspace_bytes(w.B, w.H, cap, w.d)), dtype=torch.uint8, device=dev)
        fn = lambda: fa.decode_paged(x["q"], x["k_pages"], x["v_pages"], x["block_table"],  # noqa: E731
                                     x["ctx_lens"], scale=w.scale, window=window, workspace=ws, out=o, lse=lse)
        ctx = x["ctx_lens_cpu"].to(torch.int64)
        if window is not None:
            ctx = ctx.clamp(max=window)
        work, unit = float(2 * w.Hkv * w.d * 2 * int(ctx.sum())), "GB/s"
    elif w.kind == "decode":
        o = torch.empty_like(x["q"])
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
        ws = torch.empty(max(16, fa.decode_workspace_bytes(w.B, w.H, w.L, w.d)), dtype=torch.uint8, device=dev)
        fn = lambda: fa.decode(x["q"], x["k_cache"], x["v_cache"], x["ctx_lens"], scale=w.scale,  # noqa: E731
                               workspace=ws, out=o, lse=lse, window=window)
        ctx = x["ctx_lens_cpu"].to(torch.int64)
        if window is not None:
            ctx = ctx.clamp(max=window)
        work, unit = float(2 * w.Hkv * w.d * 2 * int(ctx.sum())), "GB/s"
    elif fp8:
        o = torch.empty((w.B, w.H, w.L, w.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
        sl = x.get("seqlens")
        fn = lambda: fa.fwd_fp8(x["q"], x["k"], x["v"], x["q_descale"], x["k_descale"],  # noqa: E731
                                x["v_descale"], causal=w.causal, scale=w.scale, seqlens=sl, window=window,
                                out=o, lse=lse)
        lens = x["seqlens_cpu"].to(torch.float64) if sl is not None else torch.full((w.B,), float(w.L))
        pairs = float((lens * lens).sum()) * (0.5 if w.causal else 1.0)
        if window is not None:
            pairs = _window_pairs(lens.tolist(), window)
        work, unit = 4.0 * w.H * w.d * pairs, "TFLOP/s"
    else:
        o = torch.empty_like(x["q"])
        lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
        sl = x.get("seqlens")
        fn = lambda: fa.fwd(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale, seqlens=sl,  # noqa: E731
                            out=o, lse=lse, window=window)
        lens = x["seqlens_cpu"].to(torch.float64) if sl is not None else torch.full((w.B,), float(w.L))
        pairs = float((lens * lens).sum()) * (0.5 if w.causal else 1.0)
        if window is not None:
            pairs = _window_pairs(lens.tolist(), window)
        work, unit = 4.0 * w.H * w.d * pairs, "TFLOP/s"
    return fn, work, unit


# After an idle second the GPU runs its first launches at a low clock and takes about 40 ms of
# load to reach the clock it holds under sustained load (per-launch times of the 16k prefill
# after 2 s idle: 3.7, 2.4, 2.2, 2.1, ... ms, settling at 1.78 ms after about 20 launches). A
# change of load can take longer: FP8 prefills launched in turn with bf16 ones, right after the
# decode workload, went 1.93, 1.76, 1.68, ... 1.48, ... 1.33 ms over their first 70 ms while the
# bf16 launches beside them held steady. Every timed section therefore first runs its own
# calls untimed, back to back, each round of them bracketed by HIP events, for at least SETTLE_MS of wall
# time and then until the median round time of the last SETTLE_WINDOW rounds is no more than
# SETTLE_TOL below that of the SETTLE_WINDOW before them (the times have stopped falling), or
# SETTLE_MAX_MS has passed; then come its W warm-up launches. The figures are those of
# sustained load. The wall time each section took to settle is reported (SETTLE_LOG).
SETTLE_MS = 150.0
SETTLE_MAX_MS = 1500.0
SETTLE_WINDOW = 8
SETTLE_TOL = 0.01
SETTLE_LOG = {}


def settle(fns, label, min_ms=SETTLE_MS, max_ms=SETTLE_MAX_MS):
    """Launch the calls in turn, untimed, until the round times have stopped falling (see
    above); records the wall time taken under `label` in SETTLE_LOG. Rounds are launched back
    to back, as the timed launches are, with two rounds always queued behind the one whose
    time is read, so the GPU never idles between them: a synchronisation after every round
    left 50-70 us gaps, under which the kernels ran faster than in the back-to-back timed
    launches that followed (16k prefill: 1.77 ms settled, then 1.87 and 1.94 ms timed)."""
    import collections
    import time
    import torch
    t0 = time.perf_counter()
    rounds, queued = [], collections.deque()
    while True:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for fn in fns:
            fn()
        b.record()
        queued.append((a, b))
        if len(queued) < 3:
            continue
        a, b = queued.popleft()
        b.synchronize()
        rounds.append(a.elapsed_time(b))
        el = (time.perf_counter() - t0) * 1e3
        if el >= max_ms:
            break
        if el >= min_ms and len(rounds) >= 2 * SETTLE_WINDOW and \
                median(rounds[-SETTLE_WINDOW:]) >= (1.0 - SETTLE_TOL) * median(rounds[-2 * SETTLE_WINDOW:-SETTLE_WINDOW]):
            break
    torch.cuda.synchronize()
    SETTLE_LOG[label] = {"ms": round(el, 1), "rounds": len(rounds) + len(queued)}


def time_launches(fn, steps, warmup, label):
    """Per-launch times (ms) of `steps` launches of fn after `warmup` untimed ones, from HIP
    events on torch's current stream (the stream the kernels are launched on), after the clock
    has settled under this call's load."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    settle([fn], label)
    for _ in range(warmup):  # no synchronisation between settle, warm-ups and timed launches
        fn()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def time_interleaved(fns, steps, warmup, label, rounds=4):
    """Per-launch times (ms) of several calls timed in the same window: `rounds` rounds, each
    launching every call `steps // rounds` times in turn (after `warmup` untimed launches of
    each), so that all of them see the same clock and temperature."""
    import torch
    settle(fns, label)
    for fn in fns:
        for _ in range(warmup):
            fn()
    per = max(1, steps // rounds)
    ev = [[] for _ in fns]
    for _ in range(rounds):
        for i, fn in enumerate(fns):
            for _ in range(per):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                ev[i].append((a, b))
    torch.cuda.synchronize()
    return [[a.elapsed_time(b) for a, b in e] for e in ev]


def median(ms):
    import statistics
    return statistics.median(ms)


def workload_lines(steps, warmup, dev):
    """Each of the five workloads timed alone (bench.py's launch configuration), plus the FP8
    prefill of the 16,384-token workload. Rates come from the median launch time."""
    import fa_inputs
    out = {}
    for name, w in fa_inputs.WORKLOADS.items():
        fn, work, unit = workload_call(w, dev)
        ms = time_launches(fn, steps, warmup, name)
        med = median(ms)
        sp = spread(ms)
        if w.name == "single_head_fp32_L128_d64":
            out[name] = {"us_median": round(1e3 * med, 2), "us_p10": round(1e3 * sp["ms_p10"], 2),
                         "us_p90": round(1e3 * sp["ms_p90"], 2),
                         "note": "launch-bound (4.19 MFLOP); reported in microseconds only"}
        elif unit == "TFLOP/s":
            rate = work / (med * 1e-3) / 1e12
            tr, src = traffic_record("prefill", None if name == PREFILL else name)
            out[name] = {**sp, "tflops": round(rate, 2), "frac": round(rate / PEAK_BF16_TFLOPS, 4),
                         "flop_per_launch": work, "bound": "mfma", "peak_tflops": PEAK_BF16_TFLOPS,
                         "traffic": tr["bytes_per_launch"] if tr else None, "traffic_source": src}
        else:
            rate = work / (med * 1e-3) / 1e9
            out[name] = {**sp, "gbps": round(rate, 1), "frac": round(rate / PEAK_HBM_GBPS, 4),
                         "kv_bytes_per_launch": work, "bound": "hbm", "peak_gbps": PEAK_HBM_GBPS}
        del fn
    # The FP8 prefill and the bf16 prefill of the same workload, launched in turn in one window:
    # the speed-up compares the two kernels at the same clock and temperature.
    w = fa_inputs.WORKLOADS[PREFILL]
    fn, work, _ = workload_call(w, dev, fp8=True)
    fn_bf16, _, _ = workload_call(w, dev)
    ms, ms_bf16 = time_interleaved([fn, fn_bf16], steps, warmup, "fp8+bf16:" + PREFILL)
    med = median(ms)
    rate = work / (med * 1e-3) / 1e12
    tr, src = traffic_record("fp8")
    out["fp8:" + PREFILL] = {**spread(ms), "tflops": round(rate, 2), "frac": round(rate / PEAK_FP8_TFLOPS, 4),
                             "peak_tflops": PEAK_FP8_TFLOPS, "bound": "mfma (fp8)",
                             "bf16_ms_median_same_window": round(median(ms_bf16), 4),
                             "speedup_vs_bf16": round(median(ms_bf16) / med, 3),
                             "speedup_basis": "bf16 and FP8 prefill of this workload launched in turn, "
                                              "4 rounds, same window",
                             "kernel": "fwd_fp8_kernel (E4M3 Q/K/V, per-head descales)",
                             "traffic": tr["bytes_per_launch"] if tr else None, "traffic_source": src}
    del fn, fn_bf16
    return out


def run_only(part, steps, warmup, window=None, page=None, fp8=False):
    """Time one part alone (for profiling): the prefill or decode part of the step, a plain
    1 GiB device copy, or any named workload. Prints the kernel time and, for workloads,
    the algorithmic rate (prefill: TFLOP/s over visible pairs as in the metric; decode: K/V
    GB/s)."""
    import torch

    import exact_attention_111_amd as fa
    import fa_inputs
    dev = torch.device("cuda:0")
    name = {"prefill": PREFILL, "decode": DECODE, "backward": "backward:" + PREFILL}.get(part, part)
    rate = None
    if name.startswith("backward:") and name[len("backward:"):] in fa_inputs.WORKLOADS:
        w = fa_inputs.WORKLOADS[name[len("backward:"):]]
        if w.kind != "prefill" or w.io != "bf16":
            raise SystemExit(f"no backward for {w.name}")
        x = fa_inputs.workload_inputs(w, device=dev)
        sl = x.get("seqlens")
        o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale, seqlens=sl, window=window)
        g = torch.Generator(device=dev).manual_seed(w.seed + 1000)
        do = torch.randn(o.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        ws = torch.empty(max(16, fa.bwd_workspace_bytes(w.B, w.H, w.L)), dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
        fn = lambda: fa.bwd(x["q"], x["k"], x["v"], o, do, lse, causal=w.causal, scale=w.scale,  # noqa: E731
                            seqlens=sl, workspace=ws, dq=dq, dk=dk, dv=dv, window=window)
        lens = x["seqlens_cpu"].to(torch.float64) if sl is not None else torch.full((w.B,), float(w.L))
        pairs = float((lens * lens).sum()) * (0.5 if w.causal else 1.0)
        if window is not None:
            pairs = _window_pairs(lens.tolist(), window)
        rate = (BWD_FLOP_PER_FWD * 4.0 * w.H * w.d * pairs, "TFLOP/s")
    elif name == "copy":  # a plain copy of 1 GiB: reads 1 GiB and writes 1 GiB per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)  # noqa: E731
    elif name in fa_inputs.WORKLOADS:
        fn, work, unit = workload_call(fa_inputs.WORKLOADS[name], dev, window, page, fp8)
        rate = (work, unit)
    else:
        raise SystemExit(f"unknown part or workload: {part}")
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(); fn(); b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    line = {"only": name, "window": window, "page": page, "fp8": fp8, "steps": steps, "ms_avg": sum(ms) / len(ms), "ms_min": ms[0], "ms_median": ms[len(ms) // 2]}
    if rate is not None:
        work, unit = rate
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        line.update({"value": work / (line["ms_median"] * 1e-3) / scale, "unit": unit})
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; run with --gpus 1"}))
        sys.exit(2)
    if args.only:
        run_only(args.only, args.steps, args.warmup, args.window, args.page, args.fp8)
        return
    import torch

    import exact_attention_111_amd as fa
    import fa_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wp = fa_inputs.WORKLOADS[PREFILL]
    wd = fa_inputs.WORKLOADS[DECODE]
    xp = fa_inputs.workload_inputs(wp, device=dev)
    xd = fa_inputs.workload_inputs(wd, device=dev)
    o_p = torch.empty_like(xp["q"])
    lse_p = torch.empty((wp.B, wp.H, wp.L), dtype=torch.float32, device=dev)
    o_d = torch.empty_like(xd["q"])
    lse_d = torch.empty((wd.B, wd.H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, fa.decode_workspace_bytes(wd.B, wd.H, wd.L, wd.d)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fwd(xp["q"], xp["k"], xp["v"], causal=True, scale=wp.scale, out=o_p, lse=lse_p)
        if ev is not None:
            ev[1].record()
        fa.decode(xd["q"], xd["k_cache"], xd["v_cache"], xd["ctx_lens"], scale=wd.scale, workspace=ws, out=o_d,
                  lse=lse_d)
        if ev is not None:
            ev[2].record()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    settle([step], "step")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    fwd_med = median(fwd_ms)
    dec_med = median(dec_ms)

    # Rates from the median launch time (the mean is reported beside it).
    flop = 4.0 * wp.B * wp.H * wp.L * wp.L * wp.d / 2.0
    tflops = flop / (fwd_med * 1e-3) / 1e12
    ctx = xd["ctx_lens_cpu"].to(torch.int64)
    kv_bytes = float(2 * wd.Hkv * wd.d * 2 * int(ctx.sum()))
    gbps = kv_bytes / (dec_med * 1e-3) / 1e9

    # Backward of the same prefill (the gradients of that step for a synthetic dO), timed on
    # its own after the step: K launches of fa_bwd after W warm-up launches.
    g = torch.Generator(device=dev).manual_seed(wp.seed + 1000)
    do_p = torch.randn(o_p.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ws_b = torch.empty(max(16, fa.bwd_workspace_bytes(wp.B, wp.H, wp.L)), dtype=torch.uint8, device=dev)
    grads = (torch.empty_like(xp["q"]), torch.empty_like(xp["k"]), torch.empty_like(xp["v"]))

    def bwd_call():
        fa.bwd(xp["q"], xp["k"], xp["v"], o_p, do_p, lse_p, causal=True, scale=wp.scale, workspace=ws_b,
               dq=grads[0], dk=grads[1], dv=grads[2])

    bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    settle([bwd_call], "backward")
    for _ in range(args.warmup):
        bwd_call()
    for a_, b_ in bev:
        a_.record(); bwd_call(); b_.record()
    torch.cuda.synchronize()
    bwd_ms = [a_.elapsed_time(b_) for a_, b_ in bev]
    bwd_avg = sum(bwd_ms) / len(bwd_ms)
    bwd_flop = BWD_FLOP_PER_FWD * 4.0 * wp.B * wp.H * wp.L * wp.L * wp.d / 2.0
    bwd_tflops = bwd_flop / (median(bwd_ms) * 1e-3) / 1e12
    del grads, ws_b, do_p

    workloads = workload_lines(args.steps, args.warmup, dev)
    gemm = library_gemm_tflops(dev)

    tr_p, src_p = traffic_record("prefill")
    tr_d, src_d = traffic_record("decode")
    tr_b, src_b = traffic_record("backward")
    alg_p = float(3 * wp.B * wp.H * wp.L * wp.d * 2 + wp.B * wp.H * wp.L * wp.d * 2 + wp.B * wp.H * wp.L * 4)
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"min_ms": SETTLE_MS, "max_ms": SETTLE_MAX_MS, "window_rounds": SETTLE_WINDOW,
                   "tol": SETTLE_TOL, "taken": SETTLE_LOG},
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{PREFILL} + {DECODE}", "prefill": {"B": wp.B, "H": wp.H, "L": wp.L, "d": wp.d,
                                                                   "causal": True, "seed": wp.seed},
                   "decode": {"B": wd.B, "H": wd.H, "Hkv": wd.Hkv, "Lmax": wd.L, "d": wd.d,
                              "ctx_range": list(wd.len_range), "seed": wd.seed,
                              "ctx_sum": int(ctx.sum())}},
        "prefill": {"ms_mean": round(fwd_avg, 4), "ms_min": round(min(fwd_ms), 4), **spread(fwd_ms),
                    "tflops": round(tflops, 2),
                    "pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "flop_per_launch": flop},
        "decode": {"value": round(gbps, 1), "unit": "GB/s", "ms_mean": round(dec_avg, 4),
                   "ms_min": round(min(dec_ms), 4),
                   **spread(dec_ms),
                   "pct_hbm_peak": round(100 * gbps / PEAK_HBM_GBPS, 2), "kv_bytes_per_launch": kv_bytes},
        "backward": {"ms_mean": round(bwd_avg, 4), "ms_min": round(min(bwd_ms), 4), **spread(bwd_ms),
                     "tflops": round(bwd_tflops, 2),
                     "pct_mfma_peak": round(100 * bwd_tflops / PEAK_BF16_TFLOPS, 2), "flop_per_launch": bwd_flop,
                     "flop_counting": "5 products of the forward's size (2.5x forward FLOP)",
                     "kernels": "bwd_dot_kernel<128> + bwd_dkdv_kernel<128> + bwd_dq_kernel<128>",
                     "traffic": tr_b["bytes_per_launch"] if tr_b else None, "traffic_unit": "bytes/launch",
                     "traffic_source": src_b},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "timing": "median launch",
                     "achieved_from_mean": round(flop / (fwd_avg * 1e-3) / 1e12, 2),
                     "traffic": tr_p["bytes_per_launch"] if tr_p else None, "traffic_unit": "bytes/launch",
                     "traffic_algorithmic": alg_p, "traffic_source": src_p,
                     "kernel": "fwd_kernel<128, bf16, bf16, false>",
                     "library_gemm": gemm, "frac_of_library_gemm": round(tflops / gemm["tflops"], 4)},
        "roofline_decode": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": round(gbps / PEAK_HBM_GBPS, 4),
                            "traffic": tr_d["bytes_per_launch"] if tr_d else None, "traffic_unit": "bytes/launch",
                            "traffic_algorithmic": kv_bytes, "traffic_source": src_d,
                            "kernels": "decode_split_kernel<128, false, true> + decode_combine_kernel<128, true>"},
        "workloads": workloads,
        "context": CONTEXT,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wp, xp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
