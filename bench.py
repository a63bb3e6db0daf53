"""Benchmark: BF16 GEMM C = A * B^T at 8192^3 on one MI355X (TFLOP/s, % of 2.5 PF).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--schedule S] [--grid-order G] [--group-m G] [--window W]
                    [--no-settle] [--no-cpu-baseline] [--no-flush] [--library-context]

A step is one call of the whole path (hk_gemm_bf16 / hk_gemm_fp8 through the
C ABI) on inputs already resident in HBM.  Order of a run:

  1. settle: the step runs in windows until the chip's clock has settled
     (two consecutive windows within 1 % of each other after at least 60 ms
     of GPU time, at most 1.5 s).  After idle, MI355X boosts its clock, then
     its power controller pulls it well below the sustained level under this
     power-bound load and brings it back over some tens of milliseconds: at
     8192^3 single launches measured 0.75, 0.71, then up to 0.94 and back to
     0.69 ms over about 40 launches, the chiplet clocks 1.72, then 1.24, then
     1.70 GHz.  Any idle gap of a millisecond or so starts this again, and a
     handful of warm-up steps ends inside the dip.  Each window is queued
     before the previous one is read; the window means are under `settle`.
  2. W untimed warm-up steps, queued right behind the last settle window.
  3. exactly K timed steps back to back, bracketed by device synchronisation
     and by one pair of HIP events on the launch stream, launched as soon as
     the queue has drained, with every argument built beforehand; `value` is
     2*M*N*K*K / wall time, `roofline.achieved` uses the event time / K.
     The persistent kernels record their clocks in every timed launch
     (hk_gemm_opts.clock_stamps, which costs nothing measurable): `clock_ghz`.
  4. K more launches, each bracketed by its own events (per-launch events
     cost about 5 us of gap per launch, so they stay out of the timed
     region): `launch_ms` holds their deciles and the first ones in order.
  5. launches each preceded by a 1 GiB fill (evicting L2 and the last-level
     cache), `flushed_kernel_ms`.
  6. the CPU baseline: the FP64 oracle on a bounded sample of output rows.

`inputs` holds the SHA-256 of the operand bytes.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0}
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="bf16_8192")
    ap.add_argument("--schedule", default="auto")
    ap.add_argument("--grid-order", default="auto")
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--window", type=int, default=0)
    ap.add_argument("--no-settle", action="store_true",
                    help="skip the clock-settling launches before the warm-up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the per-launch timing after an L2/LLC flush")
    ap.add_argument("--library-context", action="store_true",
                    help="also time torch's own GEMM (hipBLASLt: torch.matmul for BF16, "
                         "torch._scaled_mm for FP8) on the same stored operands, as context")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the GEMM, run one plain device-to-device copy of BYTES "
                         "bytes (torch copy_) 5 times; the HBM byte counters read on it "
                         "calibrate those read on the GEMM")
    return ap.parse_args()


def copy_calibration(nbytes: int):
    """A plain copy kernel of known size: reads nbytes, writes nbytes per launch."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch recorded under profiles/ for this kernel source, or None.

    profiles/traffic_<kernel>_<workload>.md holds 'source_sha256: X' and
    'hbm_bytes_per_launch: Y'; the value is used only while X matches the
    current kernel sources.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m1 = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m2 = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m1 and m2):
        return None
    return (m1.group(1), float(m2.group(1))) if m1.group(1) == kernel_source_sha(kernel) else None


# The sources each kernel family is built from (its hash keys recorded traffic).
KERNEL_SOURCES = {"hk_gemm": ("hk_device.hpp", "hk_gemm.hip", "hk_grid.hpp", "hk_kernels.hpp"),
                  "hk_attn": ("hk_device.hpp", "hk_attn.hip", "hk_attn.hpp")}


def kernel_source_sha(kernel: str = "hk_gemm") -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_gemm_02_amd", "csrc")
    family = next(k for k in KERNEL_SOURCES if kernel.startswith(k))
    for f in sorted(KERNEL_SOURCES[family]):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def cpu_baseline(w, x, seconds: float):
    """The oracle, untuned, on whole output rows; scaled to TFLOP/s."""
    import numpy as np
    import oracle
    import gemm_inputs
    threads = oracle.default_threads()
    A = gemm_inputs.bits(x["A"])
    B = gemm_inputs.bits(x["B"])
    dt = "bf16" if w.dtype == "bf16" else "fp8"

    def run(rows):
        t0 = time.perf_counter()
        if w.dtype == "mxfp8":
            oracle.gemm_mx(A[:rows].ravel(), B.ravel(), x["SA"][:rows].numpy().ravel(),
                           x["SB"].numpy().ravel(), rows, w.N, w.K, threads=threads, want_s=False)
        else:
            oracle.gemm(dt, A[:rows].ravel(), B.ravel(), rows, w.N, w.K,
                        scale_a=x["scale_a"], scale_b=x["scale_b"], threads=threads, want_s=False)
        return time.perf_counter() - t0

    # calibration: one row per thread, so that the estimate sees every thread busy
    rows = max(1, threads)
    t = run(rows)
    per_row = t / rows
    rows = int(max(threads, min(w.M, seconds / max(per_row, 1e-9))))
    rows = max(threads, (rows // threads) * threads)
    t = run(rows)
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), **host_cpus(threads),
            "sample": "%d of %d output rows (all %d columns, K=%d), FP64 scalar oracle, %.1f s"
                      % (rows, w.M, w.N, w.K, t)}


def library_context(a, w, A, B, sa, sb, stream, SA=None, SB=None):
    """torch's own GEMM on the same stored operands, timed like the main launches.

    Context only: the library is hipBLASLt (torch.matmul for BF16,
    torch._scaled_mm with per-tensor scales for FP8, and with 1 x 32 E8M0
    block scales, given as the same M x K/32 and N x K/32 byte matrices, for
    MXFP8).  The logical M x K and N x K operands are views of the stored
    arrays, so a K-strided layout reaches the library as a transposed view.
    """
    import torch
    Al = A if not w.layout_a else A.t()
    Bl = B if not w.layout_b else B.t()
    out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=A.device)
    if w.dtype == "bf16":
        name = "torch.matmul (hipBLASLt)"

        def lib_step():
            torch.matmul(Al, Bl.t(), out=out)
    else:
        name = "torch._scaled_mm (hipBLASLt)"
        Al = Al.view(torch.float8_e4m3fn)  # the stored E4M3 bytes
        Bl = Bl.view(torch.float8_e4m3fn)
        if w.dtype == "mxfp8":
            name = "torch._scaled_mm, 1 x 32 E8M0 block scales (hipBLASLt)"
            ta = SA.view(torch.float8_e8m0fnu)
            tb = SB.view(torch.float8_e8m0fnu)
        else:
            ta = torch.tensor(sa, dtype=torch.float32, device=A.device)
            tb = torch.tensor(sb, dtype=torch.float32, device=A.device)

        def lib_step():
            torch._scaled_mm(Al, Bl.t(), scale_a=ta, scale_b=tb, out_dtype=torch.bfloat16,
                             out=out)
    try:
        with torch.cuda.stream(stream):
            lib_step()
        torch.cuda.synchronize()
    except RuntimeError as e:  # a storage the library does not take
        return {"library": name, "unsupported": str(e).splitlines()[0][:200]}
    with torch.cuda.stream(stream):
        for _ in range(a.warmup):
            lib_step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    with torch.cuda.stream(stream):
        for i in range(a.steps):
            starts[i].record(stream)
            lib_step()
            ends[i].record(stream)
    torch.cuda.synchronize()
    durs = sorted(s_.elapsed_time(e) for s_, e in zip(starts, ends))
    mean_ms = sum(durs) / len(durs)
    return {"library": name, "tflops": round(w.flops / (mean_ms * 1e-3) / 1e12, 2),
            "kernel_ms": {"mean": round(mean_ms, 4), "median": round(durs[len(durs) // 2], 4)}}


def settle(step, stream, min_ms: float = 60.0, max_ms: float = 1500.0, tol: float = 0.01):
    """Launch the step in windows until two consecutive window means agree.

    Stops once at least min_ms of GPU time has passed and the last two windows'
    mean launch times are within tol of each other, or after max_ms.  A window
    is at least 10 launches and about 5 ms.  The next window is always queued
    before the previous one is read, so the GPU never idles in between (an
    idle gap of a millisecond or less starts the boost and clamp again).
    Returns what it saw; the last queued window may still be running.
    """
    import torch

    def window(n):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            s.record(stream)
            for _ in range(n):
                step()
            e.record(stream)
        return s, e, n

    means, launches, gpu_ms = [], 0, 0.0
    inflight = window(10)
    while True:
        s, e, n = inflight
        inflight = window(int(min(1000, max(10, 5.0 / max(means[-1], 1e-4)))) if means else 10)
        e.synchronize()
        ms = s.elapsed_time(e)
        means.append(ms / n)
        launches += n
        gpu_ms += ms
        if gpu_ms >= max_ms:
            break
        if gpu_ms >= min_ms and len(means) >= 2 and abs(means[-1] - means[-2]) <= tol * means[-2]:
            break
    launches += inflight[2]
    return {"launches": launches, "gpu_ms_measured": round(gpu_ms, 2),
            "window_mean_ms": [round(m, 4) for m in means],
            "rule": "windows of >= 10 launches (~5 ms), each queued before the previous is read, "
                    "until two consecutive means agree within 1 %% after >= %.0f ms of GPU time, "
                    "at most %.0f ms" % (min_ms, max_ms)}


def series_events(n: int):
    import torch
    return ([torch.cuda.Event(enable_timing=True) for _ in range(n)],
            [torch.cuda.Event(enable_timing=True) for _ in range(n)])


def launch_series(step, stream, events):
    """Launches each bracketed by its own pair of (pre-built) events: durations in ms, in order.

    Queued at once after the previous synchronisation, so that the GPU idles
    as little as possible in between.
    """
    import torch
    starts, ends = events
    n = len(starts)
    with torch.cuda.stream(stream):
        for i in range(n):
            starts[i].record(stream)
            step()
            ends[i].record(stream)
    torch.cuda.synchronize()
    return [s_.elapsed_time(e) for s_, e in zip(starts, ends)]


def clock_summary(hk, stamps):
    """Mean shader clock per chiplet over the timed launches, from their clock records."""
    if stamps is None:
        return None
    khz = hk.hk_wall_clock_khz()
    rows = stamps.cpu().tolist()
    per = [hk.chiplet_clocks_ghz(r, khz) for r in rows]
    chip = []
    for x in range(8):
        v = [p[x] for p in per if p[x] is not None]
        chip.append(round(sum(v) / len(v), 3) if v else None)
    launch = [sum(c for c in p if c is not None) / max(1, sum(c is not None for c in p))
              for p in per]
    return {"per_chiplet_mean": chip,
            "launch_mean_first_last": [round(launch[0], 3), round(launch[-1], 3)],
            "mean": round(sum(launch) / len(launch), 3), "wall_clock_khz": khz,
            "how": "s_memtime / s_memrealtime spans of the first workgroup on each chiplet, "
                   "recorded by the kernel in every timed launch"}


def series_summary(durs):
    """Mean, deciles and the first launches in order, in ms."""
    srt = sorted(durs)
    q = lambda f: srt[min(len(srt) - 1, int(round(f * (len(srt) - 1))))]
    return {"launches": len(durs), "mean": round(sum(durs) / len(durs), 4),
            "min": round(srt[0], 4),
            "deciles": [round(q(i / 10.0), 4) for i in range(1, 10)],
            "max": round(srt[-1], 4),
            "first_in_order": [round(d, 4) for d in durs[:10]]}


def timed_region(step, stream, steps: int, stamps=None, before=None):
    """Exactly `steps` launches back to back: (wall seconds, event ms per launch).

    With stamps (a steps x 32 device tensor), launch i records its clocks in
    row i.  before() queues the untimed launches that precede the region; the
    region starts right after they drain, with everything it needs built.
    """
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows = [None] * steps if stamps is None else [stamps[i] for i in range(steps)]
    if before is not None:
        before()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        s.record(stream)
        if stamps is None:
            for _ in range(steps):
                step()
        else:
            for r in rows:
                step(r)
        e.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, s.elapsed_time(e) / steps


def host_cpus(threads: int) -> dict:
    """What the host offers next to the threads the oracle used."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = None
    return {"host_cpus": os.cpu_count(), "affinity_cpus": aff,
            "threads_rule": "the affinity set, capped at 16 threads (one GPU's share of the "
                            "host's cores); used %d" % threads}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only; --gpus %d is not supported: this GEMM has no "
              "multi-GPU path (an M or N split needs no exchange: run one process per GPU on its "
              "share of the output)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    import torch
    import gemm_inputs
    import fp8_gemm_02_amd as hk

    if a.workload in gemm_inputs.ATTN_WORKLOADS:
        bench_attn(a, gemm_inputs.ATTN_WORKLOADS[a.workload])
        return
    w = gemm_inputs.WORKLOADS[a.workload]
    print("[bench] workload %s M=%d N=%d K=%d %s" % (w.name, w.M, w.N, w.K, w.dtype),
          file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = gemm_inputs.make_inputs(w)
    A_st, B_st = gemm_inputs.stored(w, x)
    A = A_st.to(dev)
    B = B_st.to(dev)
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    dtype_code = {"bf16": hk.HK_DTYPE_BF16, "fp8": hk.HK_DTYPE_FP8_E4M3,
                  "mxfp8": hk.HK_DTYPE_MXFP8_E4M3}[w.dtype]
    opts = dict(schedule=a.schedule, grid_order=a.grid_order, group_m=a.group_m, window=a.window,
                layout_a=w.layout_a, layout_b=w.layout_b)
    plan = hk.hk_gemm_plan(dtype_code, A, B, C, w.M, w.N, w.K, w.lda, w.ldb, w.N, **opts)
    stream = torch.cuda.Stream()
    sa, sb = x["scale_a"], x["scale_b"]
    # digests of the logical M x K and N x K matrices (the stored arrays are
    # their transposes for a K-strided layout)
    inputs = {"A_sha256": gemm_inputs.sha256(x["A"]), "B_sha256": gemm_inputs.sha256(x["B"]),
              "scale_a": sa, "scale_b": sb}
    if w.dtype == "mxfp8":
        nb = (w.K + 31) // 32
        SA = x["SA"].to(dev)
        SB = x["SB"].to(dev)
        inputs.update(SA_sha256=gemm_inputs.sha256(x["SA"]), SB_sha256=gemm_inputs.sha256(x["SB"]))
        if a.schedule not in ("auto", "interleave4") or a.grid_order != "auto" or a.group_m or a.window:
            print("MXFP8 runs the default 4-wave kernel and order only", file=sys.stderr)
            sys.exit(2)

        def step():
            hk.hk_gemm_mxfp8(A, B, C, w.M, w.N, w.K, w.K, w.K, w.N, SA, SB, nb, nb, stream=stream)
    else:
        # operands whose rows straddle cache lines are copied to padded rows
        # first when that pays (the copy is part of every step)
        ws_bytes = hk.hk_gemm_workspace_size(dtype_code, A, B, C, w.M, w.N, w.K, w.lda, w.ldb,
                                             w.N, **opts)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        if ws_bytes:
            plan["workspace_bytes"] = ws_bytes

        def step(stamps=None):
            hk.hk_gemm_ex(dtype_code, A, B, C, w.M, w.N, w.K, w.lda, w.ldb, w.N, sa, sb,
                          stream=stream, clock_stamps=stamps, workspace=ws, **opts)

    # the persistent kernels write a clock record per launch (32 words each)
    stamps = (torch.zeros((a.steps, 32), dtype=torch.int64, device=dev)
              if w.dtype != "mxfp8" and plan["schedule"] in (hk.HK_SCHEDULE_INTERLEAVE4,
                                                              hk.HK_SCHEDULE_PINGPONG8) else None)
    print("[bench] settle, %d warm-up steps, %d timed" % (a.warmup, a.steps), file=sys.stderr,
          flush=True)
    torch.cuda.synchronize()
    settled = {}

    def before():
        # settle, then the warm-up steps queued behind its last window
        if not a.no_settle:
            settled.update(settle(step, stream))
        with torch.cuda.stream(stream):
            for _ in range(a.warmup):
                step()

    sev = series_events(a.steps)
    elapsed, event_ms = timed_region(step, stream, a.steps, stamps, before)
    series = launch_series(step, stream, sev)
    settled = settled or None
    flops = w.flops
    value = flops * a.steps / elapsed / 1e12
    achieved = flops / (event_ms * 1e-3) / 1e12

    out = {
        "metric": ("GEMM TFLOP/s at BF16 8192^3 and % of 2.5 PF BF16 peak (1 MI355X)"
                   if w.name == "bf16_8192" else
                   "GEMM TFLOP/s, %s %dx%dx%d (1 MI355X)" % (w.dtype.upper(), w.M, w.N, w.K)),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(elapsed / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "a_layout": "KxM row-major" if w.layout_a else "MxK row-major",
                   "b_layout": "KxN row-major" if w.layout_b else "NxK row-major",
                   "distribution": w.dist, "kernel": plan["kernel_name"],
                   "schedule": plan["schedule"], "grid_order": plan["grid_order"],
                   "group_m": plan["group_m"], "window": plan["window"],
                   "repacked_operands_bytes": plan.get("workspace_bytes", 0)},
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS[w.dtype], 2),
        "event_ms_per_step": round(event_ms, 4),
        "launch_ms": series_summary(series),
        "settle": settled,
        "clock_ghz": clock_summary(hk, stamps),
        "inputs": inputs,
    }
    tr = traffic_from_profiles(plan["kernel_name"], w.name)
    # The binding roofline follows the arithmetic intensity: below the ridge
    # (peak FLOP/s / peak HBM bytes/s) the shape is bound by HBM and the
    # achieved rate is algorithmic bytes per launch over the launch time.
    ai = flops / w.algorithmic_bytes
    ridge = PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2),
                           "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                           "frac": round(achieved / PEAK_TFLOPS[w.dtype], 4)}
    else:
        gbs = w.algorithmic_bytes / (event_ms * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    out["roofline"].update({"traffic": tr[1] if tr else None,
                            "arithmetic_intensity": round(ai, 1), "ridge": round(ridge, 1),
                            "algorithmic_flops_per_launch": flops,
                            "algorithmic_bytes_per_launch": w.algorithmic_bytes})

    if a.library_context:
        out["library_context"] = library_context(a, w, A, B, sa, sb, stream,
                                                 *((SA, SB) if w.dtype == "mxfp8" else ()))

    if not a.no_flush:
        # per-launch time after flushing L2 and the last-level cache (a 1 GiB
        # fill between launches, outside the events)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        fl = []
        for _ in range(max(5, a.steps // 5)):
            flush.fill_(1)
            torch.cuda.synchronize()  # the flush must finish before the timed launch
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                s.record(stream)
                step()
                e.record(stream)
            torch.cuda.synchronize()
            fl.append(s.elapsed_time(e))
        fl.sort()
        out["flushed_kernel_ms"] = {"median": round(fl[len(fl) // 2], 4), "min": round(fl[0], 4),
                                    "max": round(fl[-1], 4), "launches": len(fl)}
        del flush

    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, x, a.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_attn(w, x, seconds: float):
    """The attention oracle, untuned, on whole query rows; scaled to TFLOP/s."""
    import numpy as np
    import oracle
    import gemm_inputs
    threads = oracle.default_threads()
    q, k, v = (gemm_inputs.bits(x[n]).ravel() for n in "qkv")
    nrow = w.B * w.Hq * w.N
    rng = np.random.default_rng(0)

    def run(n):
        rows = rng.integers(0, nrow, n)
        t0 = time.perf_counter()
        oracle.attention(q, k, v, w.B, w.Hq, w.Hkv, w.N, w.D, w.scale, w.causal, rows=rows,
                         threads=threads)
        t = time.perf_counter() - t0
        keys = (rows % w.N + 1) if w.causal else np.full(n, w.N)
        return t, 4.0 * w.D * float(keys.sum())

    t, _ = run(8 * threads)  # calibration sample, large enough to amortise start-up
    n = int(max(threads, min(nrow, seconds / max(t / (8 * threads), 1e-9))))
    t, flops = run(n)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), **host_cpus(threads),
            "sample": "%d random query rows of %d (all their visible keys), FP64 scalar oracle, "
                      "%.1f s" % (n, nrow, t)}


def bench_attn(a, w):
    """Attention forward: one step is one hk_attn_fwd_bf16 launch (O and LSE)."""
    import torch
    import gemm_inputs
    import fp8_gemm_02_amd as hk
    print("[bench] workload %s B=%d Hq=%d Hkv=%d N=%d D=%d causal=%d" %
          (w.name, w.B, w.Hq, w.Hkv, w.N, w.D, w.causal), file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = gemm_inputs.make_attn_inputs(w)
    q, k, v = (x[n].to(dev) for n in "qkv")
    O = torch.empty((w.B, w.Hq, w.N, w.D), dtype=torch.bfloat16, device=dev)
    L = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    kernel = "hk_attn_fwd_d%d%s" % (w.D, "_causal" if w.causal else "")

    def step():
        hk.hk_attn_fwd_bf16(q, k, v, O, L, w.B, w.Hq, w.Hkv, w.N, w.D, w.scale, w.causal,
                            stream=stream)

    print("[bench] settle, %d warm-up steps, %d timed" % (a.warmup, a.steps), file=sys.stderr,
          flush=True)
    torch.cuda.synchronize()
    settled = {}

    def before():
        if not a.no_settle:
            settled.update(settle(step, stream))
        with torch.cuda.stream(stream):
            for _ in range(a.warmup):
                step()

    sev = series_events(a.steps)
    elapsed, event_ms = timed_region(step, stream, a.steps, None, before)
    series = launch_series(step, stream, sev)
    settled = settled or None
    value = w.flops * a.steps / elapsed / 1e12
    achieved = w.flops / (event_ms * 1e-3) / 1e12
    tr = traffic_from_profiles(kernel, w.name)
    out = {
        "metric": "attention forward TFLOP/s, BF16 B=%d Hq=%d Hkv=%d N=%d D=%d %s (1 MI355X)"
                  % (w.B, w.Hq, w.Hkv, w.N, w.D, "causal" if w.causal else "non-causal"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(elapsed / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "D": w.D,
                   "causal": w.causal, "layout": "B x H x N x D packed",
                   "distribution": "normal", "kernel": kernel,
                   "flops_counted": "4 * D per visible (query, key) pair"},
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS["bf16"], 2),
        "event_ms_per_step": round(event_ms, 4),
        "launch_ms": series_summary(series),
        "settle": settled,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": tr[1] if tr else None,
                     "arithmetic_intensity": round(w.flops / w.algorithmic_bytes, 1),
                     "algorithmic_flops_per_launch": w.flops,
                     "algorithmic_bytes_per_launch": w.algorithmic_bytes},
        "inputs": {n + "_sha256": gemm_inputs.sha256(x[n]) for n in "qkv"},
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_attn(w, x, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
