"""Benchmark of the NVFP4 FC2 hot path on one MI355X.

One step = the whole hot path on one batch of synthetic input: the fused SwiGLU ->
NVFP4 producer on gate/up [M, K] followed by the block-scaled GEMM against the
pre-quantized weight (weights are quantized once, as in inference; that launch is
timed separately and reported, not inside the step). Inputs are resident in HBM
before the timed region. Per-kernel durations come from HIP events recorded on
the stream the kernels run on (torch's current stream, which the binding passes to
the C ABI).

Prints one JSON line. `value` is the FC2 GEMM throughput, 2 * M * N * K / t_gemm with
the logical M = 37,810 (the pages count FC2 TFLOP/s this way: 5.828e12 FLOP at
15.636 ms = 372.74 TFLOP/s, "FC2 NVFP4 Scheduling Results", "Timing").

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fc2_canonical]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FC2 NVFP4 GEMM TFLOP/s (% BF16 MFMA peak) + producer GB/s @M=37810"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak (published)


def producer_bytes(m: int, k: int, swiglu: bool) -> int:
    """Algorithmic HBM bytes of the two-pass producer: inputs read twice (absmax pass,
    pack pass), QDATA and the 128-row-padded scale buffer written once."""
    m_pad = (m + 15) // 16 * 16
    s_rows = (m_pad + 127) // 128 * 128
    n_in = 2 if swiglu else 1
    return 2 * n_in * m * k * 2 + m_pad * k // 2 + s_rows * (k // 16)


def producer_single_read_bytes(m: int, k: int, swiglu: bool) -> int:
    """Algorithmic HBM bytes of the single-read producer (amax supplied): inputs read
    once, QDATA and the 128-row-padded scale buffer written once."""
    m_pad = (m + 15) // 16 * 16
    s_rows = (m_pad + 127) // 128 * 128
    n_in = 2 if swiglu else 1
    return n_in * m * k * 2 + m_pad * k // 2 + s_rows * (k // 16)


def gemm_bytes(m: int, n: int, k: int) -> int:
    """Distinct data of the GEMM: packed A and W with their scales, the padded bf16 output."""
    m_pad = (m + 15) // 16 * 16
    a = m_pad * k // 2 + (m_pad + 127) // 128 * 128 * (k // 16)
    w = n * k // 2 + (n + 127) // 128 * 128 * (k // 16)
    return a + w + m_pad * n * 2


GEMM_SOURCES = ("nvfp4_block_scaled_swiglu_amd/csrc/gemm.hip", "nvfp4_block_scaled_swiglu_amd/csrc/common.hpp")
GEMM_TRAFFIC_SUMMARY = "profiles/gemm_fc2_hbm_traffic.md"
PRODUCER_SOURCES = ("nvfp4_block_scaled_swiglu_amd/csrc/producer.hip",
                    "nvfp4_block_scaled_swiglu_amd/csrc/common.hpp")
SINGLE_READ_TRAFFIC_SUMMARY = "profiles/producer_single_read_fc2_hbm_traffic.md"
PRODUCER_TRAFFIC_SUMMARY = "profiles/producer_fc2_hbm_traffic.md"


def measured_gemm_traffic():
    return measured_traffic(GEMM_TRAFFIC_SUMMARY, GEMM_SOURCES)


def source_digest(sources) -> str:
    """sha256 of the kernel sources' code: each file with its // and /* */ comments
    removed and every run of white space collapsed to one space, so that a change of
    comments alone does not retire a summary. (The sources hold no string literal
    that contains a comment marker.)"""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()


def summary_values(summary: str, sources):
    """The value block of a committed counter summary, or None when the summary was
    taken on different kernel code than the code built here (source_digest)."""
    try:
        digest = source_digest(sources)
        vals = {}
        with open(os.path.join(ROOT, summary)) as fh:
            for line in fh:
                if ":" in line and not line.startswith(("#", "|", "`")):
                    k, _, v = line.partition(":")
                    vals[k.strip()] = v.strip()
        return vals if vals.get("source_sha256") == digest else None
    except OSError:
        return None


def measured_traffic(summary: str, sources):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by a copy kernel of known size), or None when the summary
    was taken on a different kernel source than the one built here."""
    try:
        v = summary_values(summary, sources)
        return None if v is None else int(v["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_run(summary: str, sources, work: float, peak: float, unit_scale: float):
    """Where the `traffic` figure comes from: separate rocprofv3 runs of
    `bench.py --profile-step` on this kernel source, not this process. Gives that
    command's kernel-trace time per launch and the rate and fraction of peak at that
    time (work per launch / unit_scale per second)."""
    try:
        v = summary_values(summary, sources)
        if v is None or "trace_ms_per_launch" not in v:
            return None
        ms = float(v["trace_ms_per_launch"])
        rate = work / (ms * 1e-3) / unit_scale
        return {"summary": summary, "source": "separate rocprofv3 runs (bench.py --profile-step), not this process",
                "trace_ms_per_launch": ms, "achieved_at_trace_ms": round(rate, 1),
                "frac_at_trace_ms": round(rate / peak, 4),
                "counter_run_ms_per_launch": (float(v["counter_run_ms_per_launch"])
                                              if "counter_run_ms_per_launch" in v else None)}
    except (KeyError, ValueError):
        return None


def percentiles(xs) -> dict:
    """p10 / p50 / p90 of per-launch durations (ms), nearest-rank."""
    import math
    v = sorted(xs)
    pick = lambda q: v[min(len(v) - 1, max(0, math.ceil(q * len(v)) - 1))]
    return {"p10": round(pick(0.1), 4), "p50": round(pick(0.5), 4), "p90": round(pick(0.9), 4)}


def ceilings(dev, stream) -> dict:
    """Context for the two rooflines, measured on this device: the dense fp16 MFMA rate
    with nothing but MFMAs in flight (one wave per SIMD on every CU) and the shader
    clock during it, and a plain device-to-device copy's HBM rate (read + write)."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 16384
    nv.nvfp4_mfma_ceiling(cu, 256)
    best, clocks = 0.0, []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = nv.nvfp4_mfma_ceiling(cu, iters)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = max(best, cu * 4 * iters * 4 * 2.0 * 32 * 32 * 16 / (ms * 1e-3) / 1e12)
        o = out.cpu().double()
        clocks += (o[:, 0] / (o[:, 1] / 100e6) / 1e9).tolist()
    clocks.sort()
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    stream_gbs = stream_ceilings(dev, stream)
    return {"mfma_f16_tflops": round(best, 1), "mfma_clock_ghz_p50": round(clocks[len(clocks) // 2], 3),
            "hbm_copy_gbs": round(copy_gbs, 1), **stream_gbs,
            "note": "MFMA-only kernel (4 independent v_mfma_f32_32x32x16_f16 chains per wave, one wave per "
                    "SIMD), clock from s_memtime over s_memrealtime; copy of 1 GiB, read + write bytes; "
                    "streaming probe (nvfp4_hbm_stream_ceiling: one workgroup per 16 KiB chunk, dispatched in "
                    "address order, non-temporal loads and stores) over 2 GiB reading only, and writing "
                    f"{QUANT_WRITE_SHARE:.4f} byte per byte read (the quantize launch's mix), read + write bytes"}


# bytes the quantize launch writes per byte it reads at the canonical FC2 shape
# (QDATA + padded scales over gate + up read once)
QUANT_WRITE_SHARE = (37824 * 14336 // 2 + 37888 * 896) / (2 * 37810 * 14336 * 2)


def stream_ceilings(dev, stream) -> dict:
    """The streaming probe's HBM rate reading 2 GiB alone, and reading 2 GiB while
    writing the quantize launch's share; best of 5 launches each."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    wbytes = int(nbytes * QUANT_WRITE_SHARE) // 16 * 16
    dst = torch.empty(wbytes // 4 + 4, dtype=torch.int32, device=dev)
    out = {}
    for name, wb in (("hbm_read_only_gbs", 0), ("hbm_read_write_mix_gbs", wbytes)):
        nv.nvfp4_hbm_stream_ceiling(src, nbytes, dst, wb)
        torch.cuda.synchronize()
        best = 0.0
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            written = nv.nvfp4_hbm_stream_ceiling(src, nbytes, dst, wb)
            e1.record(stream)
            torch.cuda.synchronize()
            best = max(best, (nbytes + written) / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        out[name] = round(best, 1)
    del src, dst
    return out


def gemm_clock(a, wq, d, dev, reps: int = 5, warm: int = 5) -> dict:
    """The shader clock during the GEMM: the same kernel on the same operands, launched
    through nvfp4_gemm_bf16out_clock, whose workgroups stamp their shader-clock cycles
    (s_memtime) and 100 MHz real-time ticks (s_memrealtime) from start to end. The clock
    of a workgroup is cycles / ticks x 100 MHz; p50 over the persistent workgroups of
    `reps` stamped launches. They run back to back after `warm` plain launches, with no
    host synchronisation in between (a launch after an idle gap runs slower while the
    clocks ramp), each timed with events so that its duration can be set beside the
    timed launches'."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    clks = torch.zeros((reps, 8192, 2), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warm):
        nv.nvfp4_gemm_bf16out(a, wq, out=d)
    evs = []
    for r in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        nv.nvfp4_gemm_bf16out_clock(a, wq, d, clks[r])
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ghz = []
    for r in range(reps):
        c = clks[r, : cu - cu % 8].double().cpu()
        c = c[c[:, 1] > 0]
        ghz += (c[:, 0] / (c[:, 1] / 100e6) / 1e9).tolist()
    if not ghz:
        return {"error": "no workgroup stamps"}
    ghz.sort()
    return {"ghz_p50": round(ghz[len(ghz) // 2], 3), "ghz_p10": round(ghz[len(ghz) // 10], 3),
            "ghz_p90": round(ghz[(9 * len(ghz)) // 10], 3), "workgroups": len(ghz),
            "launch_ms": [round(x.elapsed_time(y), 4) for x, y in evs],
            "source": f"nvfp4_gemm_bf16out_clock: s_memtime cycles over s_memrealtime ticks per persistent "
                      f"workgroup, same kernel and operands as the timed GEMM, {reps} launches back to back "
                      f"after {warm} plain ones"}


def producer_floor(w, ceil: dict, t_prod: float) -> dict:
    """The two-pass producer's time if each launch streamed at the probe's rate for its
    own mix: the absmax launch reads gate and up (read-only rate), the quantize launch
    reads them again and writes QDATA and scales (the read-write-mix rate)."""
    n_in = 2 if w.swiglu else 1
    read = n_in * w.m * w.k * 2
    quant = producer_single_read_bytes(w.m, w.k, w.swiglu)
    floor = read / (ceil["hbm_read_only_gbs"] * 1e6) + quant / (ceil["hbm_read_write_mix_gbs"] * 1e6)
    return {"producer_floor_ms": round(floor, 4), "producer_frac_of_floor": round(floor / t_prod, 4),
            "producer_floor_frac_of_hbm_peak": round(producer_bytes(w.m, w.k, w.swiglu) / (floor * 1e-3) / 1e9 /
                                                     PEAK_HBM_GBS, 4)}


def cold_times(run_gemm, run_producer, dev, stream, reps: int) -> dict:
    """Per-launch times with the caches cold: 1 GiB of scratch is rewritten before each
    timed launch, which evicts the 4 MB L2s and the 256 MB MALL."""
    import torch
    scratch = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    out = {}
    for name, fn in (("gemm", run_gemm), ("producer", run_producer)):
        ts = []
        for i in range(reps):
            scratch.fill_(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        out[name + "_ms"] = percentiles(ts)
    del scratch
    out["reps"] = reps
    return out


def host_cpu() -> dict:
    """What the CPU baseline runs on: logical CPUs of this process (nproc), the OS count,
    and the CPU model name as `lscpu` reports it (else /proc/cpuinfo's)."""
    import subprocess
    model, lscpu_cpus = "", None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            key, _, val = line.partition(":")
            if key.strip() == "Model name" and not model:
                model = val.strip()
            elif key.strip() == "CPU(s)" and lscpu_cpus is None and val.strip().isdigit():
                lscpu_cpus = int(val.strip())
    except (OSError, subprocess.SubprocessError):
        pass
    if not model:
        try:
            with open("/proc/cpuinfo") as fh:
                for line in fh:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return {"nproc": nproc, "os_cpu_count": os.cpu_count(), "lscpu_cpus": lscpu_cpus, "cpu_model": model}


def baseline_threads() -> int:
    """Threads for the CPU baseline: nproc, capped by OMP_NUM_THREADS when it is set (the
    share of the host's cores a one-GPU job gets)."""
    n = host_cpu()["nproc"]
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(omp))) if omp.isdigit() and int(omp) > 0 else max(1, n)


def cpu_baseline(w, threads: int, reps: int = 3) -> dict:
    """The CPU oracle, as it stands, timed on a bounded sample of the same workload:
    the exact GEMM on 4,096 evenly spaced rows (all N columns, full K), scaled to
    TFLOP/s, and the exact producer over the whole activation; the median of `reps`
    runs each (about 10-20 s of CPU work on 16 threads), plus the GEMM on 128 rows with
    one thread. The oracle is an exact-arithmetic correctness reference, not a tuned
    CPU GEMM or quantizer."""
    import statistics
    import numpy as np
    import oracle
    rows = min(4096, w.m)
    acts = w.activations(threads=threads)
    t_prod = []
    for _ in range(reps):
        t0 = time.perf_counter()
        aq, as_, ga = oracle.quantize(acts[0], acts[1] if w.swiglu else None, threads=threads)
        t_prod.append(time.perf_counter() - t0)
    del acts
    W = w.weight(threads=threads)
    wq, ws, gw = oracle.quantize(W, threads=threads)
    sel = np.arange(rows) * (w.m // rows)
    t_gemm = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.gemm_rows(aq, as_, w.m, ga, wq, ws, w.n, gw, w.k, sel, threads=threads)
        t_gemm.append(time.perf_counter() - t0)
    rows1 = min(128, w.m)
    sel1 = np.arange(rows1) * (w.m // rows1)
    t_gemm1 = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.gemm_rows(aq, as_, w.m, ga, wq, ws, w.n, gw, w.k, sel1, threads=1)
        t_gemm1.append(time.perf_counter() - t0)
    tg, tp, tg1 = statistics.median(t_gemm), statistics.median(t_prod), statistics.median(t_gemm1)
    return {
        "value": 2.0 * rows * w.n * w.k / tg / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"median of {reps}: exact int64 GEMM of {rows} rows (every {w.m // rows}th of {w.m}) x {w.n} x "
                  f"{w.k} ({tg:.2f} s; all {w.m} rows extrapolated: {tg * w.m / rows:.1f} s); exact producer over "
                  f"all {w.m} x {w.k}: {producer_bytes(w.m, w.k, w.swiglu) / tp / 1e9:.3f} GB/s ({tp:.2f} s)",
        "host": dict(host_cpu(), threads_used=threads),
        "note": "the oracle is an exact-arithmetic correctness reference, not a tuned CPU GEMM or quantizer",
        "single_thread": {"value": 2.0 * rows1 * w.n * w.k / tg1 / 1e12, "unit": "TFLOP/s",
                          "sample": f"median of {reps}: exact GEMM of {rows1} evenly spaced rows on 1 thread "
                                    f"({tg1:.2f} s)"},
    }


def only_gemm(w, args, dev) -> int:
    """GEMM-only timing on seeded random operand bytes: QDATA uniform over all 256 byte
    values, scale bytes uniform in [0x30, 0x47] (0.5 .. 15), global scales 1."""
    import statistics
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    import synth
    tensors = []
    for rows, tag in ((w.m, 101), (w.n, 102)):
        t = nv.empty_nvfp4(rows, w.k, dev)
        t.qdata.copy_(torch.from_numpy(synth.uniform_bytes(t.qdata.numel(), w.seed, tag)).view(t.qdata.shape))
        t.scales.copy_(torch.from_numpy(synth.uniform_bytes(t.scales.numel(), w.seed, tag + 10, 0x30, 0x47)))
        t.global_scale.fill_(1.0)
        tensors.append(t)
    a, wq = tensors
    d = torch.empty((w.m_pad, w.n), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        nv.nvfp4_gemm_bf16out(a, wq, out=d)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        nv.nvfp4_gemm_bf16out(a, wq, out=d)
        e[1].record(stream)
    torch.cuda.synchronize()
    t_gemm = statistics.fmean(e[0].elapsed_time(e[1]) for e in evs)
    tflops = w.gemm_flops / (t_gemm * 1e-3) / 1e12
    out = {"mode": "only-gemm (random operand bytes)", "workload": w.name, "gemm_ms": round(t_gemm, 4),
           "tflops": round(tflops, 2), "frac_of_peak": round(tflops / PEAK_MFMA_TFLOPS, 4), "steps": args.steps,
           "gemm_distinct_bytes": gemm_bytes(w.m, w.n, w.k)}
    if args.copy_bytes > 0:
        out.update(copy_calibration(args.copy_bytes, args.steps, dev, stream))
    print(json.dumps(out), flush=True)
    return 0


def copy_calibration(nbytes: int, steps: int, dev, stream) -> dict:
    """Calibration for the profiler's byte counters: a plain elementwise pass that reads
    nbytes and writes nbytes (int32 x | 0), launched `steps` times."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.bitwise_or(src, 0, out=dst)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(steps):
        torch.bitwise_or(src, 0, out=dst)
    c1.record(stream)
    torch.cuda.synchronize()
    t_copy = c0.elapsed_time(c1) / steps
    return {"copy_bytes": 4 * n, "copy_ms": round(t_copy, 4), "copy_gbs": round(2 * 4 * n / (t_copy * 1e-3) / 1e9, 1)}


def profile_step(w, args, dev) -> int:
    """The bench's timed step alone: the producer and the GEMM on the workload's seeded
    inputs (the weight quantized once before), warm-up and timed steps exactly as in the
    default run, and nothing else launched afterwards except the optional copy
    calibration. This is the command the profiler traces and counts, so that its
    per-kernel averages describe the same launches as the bench line's `producer_ms`
    and `gemm_ms`. Prints one JSON line with the HIP-event averages."""
    import statistics
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    from tests import parity
    acts = w.activations()
    x = parity.to_device_bf16(acts[0], dev)
    u = parity.to_device_bf16(acts[1], dev) if w.swiglu else None
    del acts
    wt = parity.to_device_bf16(w.weight(), dev)
    a = nv.empty_nvfp4(w.m, w.k, dev)
    wq = nv.empty_nvfp4(w.n, w.k, dev)
    d = torch.empty((w.m_pad, w.n), dtype=torch.bfloat16, device=dev)
    nv.nvfp4_quantize(wt, out=wq)
    del wt
    stream = torch.cuda.current_stream()

    def producer():
        if w.swiglu:
            nv.nvfp4_quantize_swiglu(x, u, out=a)
        else:
            nv.nvfp4_quantize(x, out=a)

    for _ in range(args.warmup):
        producer()
        nv.nvfp4_gemm_bf16out(a, wq, out=d)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        producer()
        e[1].record(stream)
        nv.nvfp4_gemm_bf16out(a, wq, out=d)
        e[2].record(stream)
    torch.cuda.synchronize()
    t_prod = statistics.fmean(e[0].elapsed_time(e[1]) for e in evs)
    t_gemm = statistics.fmean(e[1].elapsed_time(e[2]) for e in evs)
    clock = gemm_clock(a, wq, d, dev)  # after the timed launches: 5 warm, then 5 stamped
    out = {"mode": "profile-step", "workload": w.name, "steps": args.steps, "warmup": args.warmup,
           "gemm_clock": clock,
           "producer_ms": round(t_prod, 4), "gemm_ms": round(t_gemm, 4),
           "gemm_tflops": round(w.gemm_flops / (t_gemm * 1e-3) / 1e12, 2),
           "producer_gbs": round(producer_bytes(w.m, w.k, w.swiglu) / (t_prod * 1e-3) / 1e9, 1),
           "dispatches_per_kernel": args.warmup + args.steps,
           "note": "the activation producer is two launches (absmax, then quantize); the weight's plain "
                   "quantization (one absmax and one quantize launch of the plain kernels) runs once before; "
                   "5 clock-stamped GEMM launches follow the timed steps"}
    if args.copy_bytes > 0:
        out.update(copy_calibration(args.copy_bytes, args.steps, dev, stream))
    print(json.dumps(out), flush=True)
    return 0


def only_producer(w, args, dev) -> int:
    """Producer-only timing on the workload's seeded inputs (no GEMM in the process).
    With --single-read, the single-read producer alone, with the amax an upstream stage
    would supply (set up with the library's silu, not timed)."""
    import statistics
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    from tests import parity
    acts = w.activations()
    x = parity.to_device_bf16(acts[0], dev)
    u = parity.to_device_bf16(acts[1], dev) if w.swiglu else None
    del acts
    a = nv.empty_nvfp4(w.m, w.k, dev)
    stream = torch.cuda.current_stream()
    amax = None
    if args.single_read:
        if w.swiglu:
            sx = nv.nvfp4_silu_bf16(x.view(torch.int16)).view(torch.bfloat16)
            amax = (sx.float() * u.float()).bfloat16().abs().max().float().reshape(1)
            del sx
        else:
            amax = x.abs().max().float().reshape(1)
        torch.cuda.synchronize()

    def run():
        if amax is not None:
            if w.swiglu:
                nv.nvfp4_quantize_swiglu_amax(x, u, amax, out=a)
            else:
                nv.nvfp4_quantize_amax(x, amax, out=a)
        elif w.swiglu:
            nv.nvfp4_quantize_swiglu(x, u, out=a)
        else:
            nv.nvfp4_quantize(x, out=a)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    t_prod = statistics.fmean(e[0].elapsed_time(e[1]) for e in evs)
    pbytes = (producer_single_read_bytes if args.single_read else producer_bytes)(w.m, w.k, w.swiglu)
    out = {"mode": "only-producer" + (" (single read)" if args.single_read else ""), "workload": w.name,
           "producer_ms": round(t_prod, 4), "gbs": round(pbytes / (t_prod * 1e-3) / 1e9, 1),
           "algorithmic_bytes": pbytes, "steps": args.steps}
    if args.copy_bytes > 0:
        out.update(copy_calibration(args.copy_bytes, args.steps, dev, stream))
    print(json.dumps(out), flush=True)
    return 0


SHAPES = ("fc2_canonical", "qkv", "qkv_pages", "attn_out", "fc1")


def shapes(args, dev) -> int:
    """Producer + GEMM on each projection shape (seeded inputs of that shape; weights
    quantized once outside the timing). One JSON line per shape."""
    import statistics
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    import synth
    from tests import parity
    stream = torch.cuda.current_stream()
    for name in SHAPES:
        w = synth.BY_NAME[name]
        acts = w.activations()
        x = parity.to_device_bf16(acts[0], dev)
        u = parity.to_device_bf16(acts[1], dev) if w.swiglu else None
        del acts
        wt = parity.to_device_bf16(w.weight(), dev)
        a = nv.empty_nvfp4(w.m, w.k, dev)
        wq = nv.empty_nvfp4(w.n, w.k, dev)
        nv.nvfp4_quantize(wt, out=wq)
        d = torch.empty((w.m_pad, w.n), dtype=torch.bfloat16, device=dev)

        def producer():
            if w.swiglu:
                nv.nvfp4_quantize_swiglu(x, u, out=a)
            else:
                nv.nvfp4_quantize(x, out=a)

        for _ in range(args.warmup):
            producer()
            nv.nvfp4_gemm_bf16out(a, wq, out=d)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for e in evs:
            e[0].record(stream)
            producer()
            e[1].record(stream)
            nv.nvfp4_gemm_bf16out(a, wq, out=d)
            e[2].record(stream)
        torch.cuda.synchronize()
        t_prod = statistics.fmean(e[0].elapsed_time(e[1]) for e in evs)
        t_gemm = statistics.fmean(e[1].elapsed_time(e[2]) for e in evs)
        t_mod = None
        if not w.swiglu:
            # the same input with adaLN modulation fused into the quantizer
            sc = (torch.randn(w.k, device=dev) * 0.3).bfloat16()
            sh = (torch.randn(w.k, device=dev) * 0.5).bfloat16()
            nv.nvfp4_quantize_modulate(x, sc, sh, out=a)
            torch.cuda.synchronize()
            evm = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            for e in evm:
                e[0].record(stream)
                nv.nvfp4_quantize_modulate(x, sc, sh, out=a)
                e[1].record(stream)
            torch.cuda.synchronize()
            t_mod = statistics.fmean(e[0].elapsed_time(e[1]) for e in evm)
        tflops = w.gemm_flops / (t_gemm * 1e-3) / 1e12
        pbytes = producer_bytes(w.m, w.k, w.swiglu)
        print(json.dumps({"mode": "shapes", "workload": name, "m": w.m, "n": w.n, "k": w.k,
                          "producer": "swiglu" if w.swiglu else "plain", "producer_ms": round(t_prod, 4),
                          "producer_gbs": round(pbytes / (t_prod * 1e-3) / 1e9, 1), "gemm_ms": round(t_gemm, 4),
                          "gemm_tflops": round(tflops, 2), "gemm_frac_of_peak": round(tflops / PEAK_MFMA_TFLOPS, 4),
                          "producer_modulate_ms": None if t_mod is None else round(t_mod, 4),
                          "steps": args.steps}), flush=True)
        del x, u, wt, a, wq, d
        torch.cuda.empty_cache()
    return 0


def chain(args, dev) -> int:
    """The MLP block with every fusion, on the FC1 and FC2 shapes (M = 37,810):
      modulated quantize (f2) -> FC1 SwiGLU-pair GEMM emitting amax (f3)
      -> single-read FC2 producer (f1) -> FC2 GEMM with bias + gated residual (f3),
    against the unfused path on the same operands: the adaLN modulation as its own
    elementwise kernel, plain quantize, FC1 GEMM, two-pass FC2 producer, FC2 GEMM,
    then the bias add and the gated residual add as elementwise kernels. The unfused
    path's elementwise steps are torch's kernels (they are what the fusions remove,
    not steps of this library). Weights are quantized once, outside the timing; the
    modulation, bias, gate and residual are seeded."""
    import statistics
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    import synth
    from tests import parity
    w1, w2 = synth.BY_NAME["fc1"], synth.FC2
    m, k1, nh, n2 = w1.m, w1.k, w1.n // 2, w2.n
    g = torch.Generator(device="cpu").manual_seed(5)
    x = parity.to_device_bf16(w1.activations()[0], dev)
    W1 = parity.to_device_bf16(w1.weight(), dev)
    W1i = nv.interleave_swiglu_weight(W1[:nh], W1[nh:]).contiguous()
    w1q = nv.nvfp4_quantize(W1)      # unfused FC1: gate rows, then up rows
    w1qi = nv.nvfp4_quantize(W1i)    # SwiGLU-pair FC1: rows interleaved in chunks of 8
    del W1, W1i
    W2 = parity.to_device_bf16(w2.weight(), dev)
    w2q = nv.nvfp4_quantize(W2)
    del W2
    sc = (torch.randn(k1, generator=g) * 0.3).bfloat16().to(dev)
    sh = (torch.randn(k1, generator=g) * 0.5).bfloat16().to(dev)
    sc1 = (1.0 + sc.float()).bfloat16()
    bias2 = (torch.randn(n2, generator=g) * 0.1).bfloat16().to(dev)
    gate2 = (torch.randn(n2, generator=g) * 0.7).bfloat16().to(dev)
    m_pad = nv.nvfp4_padded_rows(m)
    res = (torch.randn(m_pad, n2, generator=g) * 0.3).bfloat16().to(dev)
    xm = torch.empty_like(x)  # the unfused path's modulated input
    a1 = nv.empty_nvfp4(m, k1, dev)
    a2 = nv.empty_nvfp4(m, nh, dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    gate_o = torch.empty((m_pad, nh), dtype=torch.bfloat16, device=dev)
    up_o = torch.empty_like(gate_o)
    d1 = torch.empty((m_pad, 2 * nh), dtype=torch.bfloat16, device=dev)
    d2 = torch.empty((m_pad, n2), dtype=torch.bfloat16, device=dev)
    o2 = torch.empty_like(d2)
    stream = torch.cuda.current_stream()

    fused_names = ["modulate_quantize", "fc1_gemm", "fc2_producer", "fc2_gemm"]

    def fused(ev):
        ev[0].record(stream)
        nv.nvfp4_quantize_modulate(x, sc, sh, out=a1)
        ev[1].record(stream)
        amax.zero_()
        nv.nvfp4_gemm_swiglu_pair(a1, w1qi, amax=amax, amax_rows=m, gate_out=gate_o, up_out=up_o)
        ev[2].record(stream)
        nv.nvfp4_quantize_swiglu_amax(gate_o[:m], up_o[:m], amax, out=a2)
        ev[3].record(stream)
        nv.nvfp4_gemm_bf16out_fused(a2, w2q, bias=bias2, gate=gate2, residual=res, out=d2)
        ev[4].record(stream)

    unfused_names = ["modulate", "quantize", "fc1_gemm", "fc2_producer", "fc2_gemm", "bias_add", "gated_residual"]

    def unfused(ev):
        ev[0].record(stream)
        torch.addcmul(sh, x, sc1, out=xm)
        ev[1].record(stream)
        nv.nvfp4_quantize(xm, out=a1)
        ev[2].record(stream)
        nv.nvfp4_gemm_bf16out(a1, w1q, out=d1)
        ev[3].record(stream)
        nv.nvfp4_quantize_swiglu(d1[:m, :nh], d1[:m, nh:], out=a2)
        ev[4].record(stream)
        nv.nvfp4_gemm_bf16out(a2, w2q, out=d2)
        ev[5].record(stream)
        d2.add_(bias2)
        ev[6].record(stream)
        torch.addcmul(res, d2, gate2, out=o2)
        ev[7].record(stream)

    out = {"mode": "chain", "m": m, "fc1": [2 * nh, k1], "fc2": [n2, nh], "steps": args.steps}
    for label, fn, names in (("fused", fused, fused_names), ("unfused", unfused, unfused_names)):
        ne = len(names) + 1
        for _ in range(max(1, args.warmup)):
            fn([torch.cuda.Event(enable_timing=True) for _ in range(ne)])
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ne)] for _ in range(args.steps)]
        for ev in evs:
            fn(ev)
        torch.cuda.synchronize()
        parts = {nm: round(statistics.fmean(ev[i].elapsed_time(ev[i + 1]) for ev in evs), 4)
                 for i, nm in enumerate(names)}
        parts["total_ms"] = round(sum(parts[nm] for nm in names), 4)
        out[label] = parts
    out["fused_over_unfused"] = round(out["fused"]["total_ms"] / out["unfused"]["total_ms"], 4)
    out["note"] = ("fused: modulate+quantize, FC1 SwiGLU-pair GEMM emitting amax, single-read FC2 producer, "
                   "FC2 GEMM with bias and gated residual; unfused: modulation, plain quantize, FC1 GEMM, two-pass "
                   "FC2 producer, FC2 GEMM, bias add, gated residual add (the three elementwise steps are torch "
                   "kernels)")
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fc2_canonical")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-gemm", action="store_true",
                    help="time the GEMM alone on seeded random NVFP4 operand bytes (no producer launch in "
                         "the process; used for profiler counter runs)")
    ap.add_argument("--chain", action="store_true",
                    help="the MLP block with every fusion against the unfused path, one JSON line")
    ap.add_argument("--shapes", action="store_true",
                    help="producer + GEMM on every projection shape, one JSON line each")
    ap.add_argument("--only-producer", action="store_true",
                    help="time the producer alone on the workload's seeded inputs (no GEMM launch)")
    ap.add_argument("--single-read", action="store_true",
                    help="with --only-producer: time the single-read producer (amax supplied) instead")
    ap.add_argument("--profile-step", action="store_true",
                    help="the timed step alone (producer + GEMM), for profiler traces and counter runs")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="with --only-gemm, --only-producer or --profile-step: also run a plain elementwise copy "
                         "of this many "
                         "bytes (read + write), the calibration kernel for the profiler's FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path runs on a single GPU (one GPU's share of an "
              f"M-sharded job); got --gpus {args.gpus}", file=sys.stderr)
        return 2

    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    import synth
    from tests import parity

    w = synth.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nv.nvfp4_init()

    if args.only_gemm:
        return only_gemm(w, args, dev)
    if args.only_producer:
        return only_producer(w, args, dev)
    if args.profile_step:
        return profile_step(w, args, dev)
    if args.shapes:
        return shapes(args, dev)
    if args.chain:
        return chain(args, dev)

    t0 = time.perf_counter()
    acts = w.activations()
    W = w.weight()
    x = parity.to_device_bf16(acts[0], dev)
    u = parity.to_device_bf16(acts[1], dev) if w.swiglu else None
    wt = parity.to_device_bf16(W, dev)
    del acts, W
    a = nv.empty_nvfp4(w.m, w.k, dev)
    wq = nv.empty_nvfp4(w.n, w.k, dev)
    d = torch.empty((w.m_pad, w.n), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0

    stream = torch.cuda.current_stream()

    # weight quantization: once, outside the step (first call warms the kernel)
    nv.nvfp4_quantize(wt, out=wq)
    ev_w0, ev_w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev_w0.record(stream)
    nv.nvfp4_quantize(wt, out=wq)
    ev_w1.record(stream)

    def step():
        if w.swiglu:
            nv.nvfp4_quantize_swiglu(x, u, out=a)
        else:
            nv.nvfp4_quantize(x, out=a)
        nv.nvfp4_gemm_bf16out(a, wq, out=d)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        if w.swiglu:
            nv.nvfp4_quantize_swiglu(x, u, out=a)
        else:
            nv.nvfp4_quantize(x, out=a)
        evs[i][1].record(stream)
        nv.nvfp4_gemm_bf16out(a, wq, out=d)
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the single-read producer (caller-supplied amax): timed after the step loop on the
    # same inputs. amax = max |y| as an upstream stage would produce it: the library's
    # bf16 silu, the exact fp32 product, one rounding to bf16 (set-up, not timed).
    if w.swiglu:
        sx = nv.nvfp4_silu_bf16(x.view(torch.int16)).view(torch.bfloat16)
        amax = (sx.float() * u.float()).bfloat16().abs().max().float().reshape(1)
        del sx
    else:
        amax = x.abs().max().float().reshape(1)
    a1 = nv.empty_nvfp4(w.m, w.k, dev)

    def single_read():
        if w.swiglu:
            nv.nvfp4_quantize_swiglu_amax(x, u, amax, out=a1)
        else:
            nv.nvfp4_quantize_amax(x, amax, out=a1)

    single_read()
    torch.cuda.synchronize()
    evs1 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evs1:
        e[0].record(stream)
        single_read()
        e[1].record(stream)
    torch.cuda.synchronize()
    same_bytes = bool(torch.equal(a1.qdata, a.qdata) and torch.equal(a1.scales, a.scales))

    # the fused epilogue (bias, gate, residual in place of the plain store), timed the
    # same way on the same operands: its cost over the plain GEMM is the epilogue's
    bias_t = (torch.randn(w.n, device=dev) * 0.5).bfloat16()
    gate_t = (torch.randn(w.n, device=dev) * 0.7).bfloat16()
    res_t = (torch.randn(w.m_pad, w.n, device=dev) * 0.3).bfloat16()
    d_f = torch.empty_like(d)
    nv.nvfp4_gemm_bf16out_fused(a, wq, bias=bias_t, gate=gate_t, residual=res_t, out=d_f)
    torch.cuda.synchronize()
    evs2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evs2:
        e[0].record(stream)
        nv.nvfp4_gemm_bf16out_fused(a, wq, bias=bias_t, gate=gate_t, residual=res_t, out=d_f)
        e[1].record(stream)
    torch.cuda.synchronize()
    del res_t, d_f

    prod_ms = [e[0].elapsed_time(e[1]) for e in evs]
    gemm_ms = [e[1].elapsed_time(e[2]) for e in evs]

    def producer_once():
        if w.swiglu:
            nv.nvfp4_quantize_swiglu(x, u, out=a)
        else:
            nv.nvfp4_quantize(x, out=a)

    cold = cold_times(lambda: nv.nvfp4_gemm_bf16out(a, wq, out=d), producer_once, dev, stream,
                      min(args.steps, 10))
    ceil = ceilings(dev, stream)
    clock = gemm_clock(a, wq, d, dev)
    import statistics
    t_prod = statistics.fmean(prod_ms)
    t_gemm = statistics.fmean(gemm_ms)
    t_single = statistics.fmean(e[0].elapsed_time(e[1]) for e in evs1)
    t_fused = statistics.fmean(e[0].elapsed_time(e[1]) for e in evs2)
    sbytes = producer_single_read_bytes(w.m, w.k, w.swiglu)
    ms_per_step = wall * 1e3 / args.steps
    tflops = w.gemm_flops / (t_gemm * 1e-3) / 1e12
    pbytes = producer_bytes(w.m, w.k, w.swiglu)
    prod_gbs = pbytes / (t_prod * 1e-3) / 1e9
    finite = bool(torch.isfinite(d[: w.m].float()).all().item())

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: SwiGLU->NVFP4 producer + NVFP4 GEMM, M={w.m} (padded {w.m_pad}), "
                        f"N={w.n}, K={w.k}, seed {w.seed}" if w.swiglu else
                        f"{w.name}: NVFP4 quantize + NVFP4 GEMM, M={w.m}, N={w.n}, K={w.k}, seed {w.seed}",
            "m": w.m, "m_padded": w.m_pad, "n": w.n, "k": w.k, "seed": w.seed,
            "outlier_channels": w.n_outliers,
            "operands": "E2M1 + vector-16 UE4M3 scales + fp32 global scale, dequantized exactly to fp16 "
                        "for fp16 MFMA, fp32 accumulation, bf16 output",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
            "traffic": measured_gemm_traffic() if w.name == "fc2_canonical" else None,
            "traffic_summary": GEMM_TRAFFIC_SUMMARY,
            "traffic_run": (traffic_run(GEMM_TRAFFIC_SUMMARY, GEMM_SOURCES, w.gemm_flops, PEAK_MFMA_TFLOPS, 1e12)
                            if w.name == "fc2_canonical" else None),
            "kernel": "nvfp4::gemm_kernel<0>",
            "algorithmic_per_launch": f"{w.gemm_flops:.4e} FLOP (2*M*N*K, logical M)",
            "avg_launch_ms": round(t_gemm, 4),
        },
        "roofline_producer": {
            "bound": "hbm",
            "achieved": round(prod_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(prod_gbs / PEAK_HBM_GBS, 4),
            "traffic": (measured_traffic(PRODUCER_TRAFFIC_SUMMARY, PRODUCER_SOURCES)
                        if w.name == "fc2_canonical" else None),
            "traffic_summary": PRODUCER_TRAFFIC_SUMMARY,
            "traffic_run": (traffic_run(PRODUCER_TRAFFIC_SUMMARY, PRODUCER_SOURCES, pbytes, PEAK_HBM_GBS, 1e9)
                            if w.name == "fc2_canonical" else None),
            "kernel": ("nvfp4::producer_absmax_kernel<1> then nvfp4::producer_kernel<1, false>" if w.swiglu else
                       "nvfp4::producer_absmax_kernel<0> then nvfp4::producer_kernel<0, false>"),
            "algorithmic_per_launch": f"{pbytes} B per call of its two launches (inputs read twice, QDATA + "
                                      f"padded scales written)",
            "avg_launch_ms": round(t_prod, 4),
        },
        "producer_single_read": {
            "entry": "nvfp4_quantize_swiglu_amax" if w.swiglu else "nvfp4_quantize_amax",
            "avg_launch_ms": round(t_single, 4),
            "algorithmic_per_launch": f"{sbytes} B (inputs read once, QDATA + padded scales written)",
            "achieved_gbs": round(sbytes / (t_single * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(sbytes / (t_single * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_equal_two_pass": same_bytes,
            "traffic": (measured_traffic(SINGLE_READ_TRAFFIC_SUMMARY, PRODUCER_SOURCES)
                        if w.name == "fc2_canonical" else None),
            "traffic_summary": SINGLE_READ_TRAFFIC_SUMMARY,
        },
        "gemm_fused_epilogue": {
            "entry": "nvfp4_gemm_bf16out_fused",
            "epilogue": "bias[n] before the rounding, then residual + gate[n] * D1",
            "avg_launch_ms": round(t_fused, 4),
            "tflops": round(w.gemm_flops / (t_fused * 1e-3) / 1e12, 2),
            "over_plain_ms": round(t_fused - t_gemm, 4),
        },
        "producer_ms": round(t_prod, 4),
        "gemm_ms": round(t_gemm, 4),
        "warm_ms": {"gemm": percentiles(gemm_ms), "producer": percentiles(prod_ms)},
        "cold_ms": cold,
        "ceilings": dict(ceil, gemm_frac_of_mfma_ceiling=round(tflops / ceil["mfma_f16_tflops"], 4),
                         producer_frac_of_copy=round(prod_gbs / ceil["hbm_copy_gbs"], 4),
                         **producer_floor(w, ceil, t_prod)),
        "gemm_clock": clock,
        "step_tflops": round(w.gemm_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "weight_quantize_ms": round(ev_w0.elapsed_time(ev_w1), 4),
        "gemm_distinct_bytes": gemm_bytes(w.m, w.n, w.k),
        "output_finite": finite,
        "setup_s": round(setup_s, 1),
        "device": torch.cuda.get_device_name(dev),
        "build": nv.nvfp4_build_info(),
    }
    if not args.no_cpu_baseline:
        threads = baseline_threads()
        try:
            line["cpu_baseline"] = cpu_baseline(w, threads)
        except Exception as e:  # the baseline is a report, not the product
            line["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
