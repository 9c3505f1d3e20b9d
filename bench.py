#!/usr/bin/env python3
"""Benchmark of the band -> bidiagonal reduction on one MI355X.

One step = one full reduction (pack, every pass, extract) of the workload's
band, already resident in device memory when the timed region starts.

Prints one JSON line:
  metric / unit   effective GB/s = algorithmic bytes of the reduction / time
                  (ms per reduction is ms_per_step)
  roofline        the dominant kernel's algorithmic bytes per launch over its
                  average launch duration (HIP events on the stream the
                  kernels run on), against the published HBM3E peak
  cpu_baseline    the CPU oracle (one thread) timed on a bounded prefix of the
                  same reduction, in the same unit

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bb_inputs  # noqa: E402

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def pass_list(bw, tw):
    out, b = [], bw
    while b > 1:
        t = min(tw, b - 1)
        out.append((b, t))
        b -= t
    return out


def alg_bytes_prefix(n, bw, tw, esize, ncycles):
    """Algorithmic bytes of the first `ncycles` cycles in sequential order."""
    total, left = 0.0, ncycles
    for (b, t) in pass_list(bw, tw):
        if left <= 0:
            break
        bp = b - t
        R = np.arange(max(n - bp - 1, 0), dtype=np.int64)
        K = (n - 2 - R - bp) // b + 1
        Rr = np.repeat(R, K)
        k = np.arange(Rr.size, dtype=np.int64) - np.repeat(np.cumsum(K) - K, K)
        take = min(left, Rr.size)
        Rr, k = Rr[:take], k[:take]
        c = Rr + bp + k * b
        ch = np.minimum(c + t, n - 1)
        r = np.where(k == 0, Rr, c - b)
        m = ch - c + 1
        rows = ch - r + 1
        cols = np.minimum(c + t + b, n - 1) - c + 1
        total += float(np.sum(2.0 * m * (rows + cols - m) * esize))
        left -= take
    return total


def cpu_baseline(band, w, seconds):
    import oracle
    oracle.build()
    esize = 8 if w.dtype == "f64" else 4
    # calibrate on a short prefix, then size the sample to about `seconds`
    t0 = time.perf_counter()
    _, _, done = oracle.reduce(band, w.bw, w.tw, max_cycles=100000)
    dt = time.perf_counter() - t0
    rate = alg_bytes_prefix(w.n, w.bw, w.tw, esize, done) / max(dt, 1e-9)
    target = rate * seconds
    # grow the cycle count until the prefix holds about `target` bytes
    ncyc = done
    while alg_bytes_prefix(w.n, w.bw, w.tw, esize, ncyc * 2) < target and ncyc < 10 ** 9:
        ncyc *= 2
    t0 = time.perf_counter()
    _, _, done = oracle.reduce(band, w.bw, w.tw, max_cycles=ncyc)
    dt = time.perf_counter() - t0
    nbytes = alg_bytes_prefix(w.n, w.bw, w.tw, esize, done)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of the reduction's cycles in sequential order "
                      f"({nbytes / 1e9:.2f} GB algorithmic, {dt:.1f} s, one thread)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=bb_inputs.HEADLINE)
    ap.add_argument("--scheduler", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this reduction runs on one GPU: one matrix is one dependent chain of "
                                   "sweeps; --gpus above 1 is not supported"}))
        sys.exit(2)

    import torch
    import band_bidiagonal_bulge_amd as bbm

    w = bb_inputs.WORKLOADS[args.workload]
    band = bb_inputs.make_workload(w)
    dev = torch.device("cuda:0")
    tb = torch.from_numpy(band).to(dev)
    dt = bbm.dtype_code(tb.dtype)
    info = bbm.bb_plan(w.n, w.bw, w.tw, dt)
    work = bbm.workspace(w.n, w.bw, w.tw, tb.dtype, dev)
    d = torch.empty(w.n, dtype=tb.dtype, device=dev)
    e = torch.empty(w.n - 1, dtype=tb.dtype, device=dev)
    tun = bbm.tuning(scheduler=args.scheduler)
    stream = torch.cuda.current_stream(dev)

    def one():
        bbm.bb_reduce(tb.data_ptr(), tb.stride(0), w.n, w.bw, w.tw, dt, d.data_ptr(), e.data_ptr(),
                      work.data_ptr(), work.numel(), tun, stream.cuda_stream)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s, f in evs:
        s.record(stream)
        one()
        f.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = [s.elapsed_time(f) for s, f in evs]
    ms_per_step = wall * 1e3 / args.steps
    value = info.alg_bytes / (ms_per_step * 1e-3) / 1e9
    kern_ms = statistics.median(ev_ms)
    achieved = info.alg_bytes / (kern_ms * 1e-3) / 1e9
    status = bbm.bb_device_status(work.data_ptr(), w.n, w.bw, w.tw, dt, stream.cuda_stream)

    out = {
        "metric": "effective GB/s (algorithmic bytes / time), band->bidiagonal n=16384 BW=64 TW=16 fp32"
        if args.workload == bb_inputs.HEADLINE else f"effective GB/s, {args.workload}",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "bw": w.bw, "tw": w.tw, "dist": w.dist, "seed": w.seed,
                   "passes": info.passes, "cycles": info.cycles, "alg_bytes": info.alg_bytes,
                   "scheduler": args.scheduler},
        "ms_per_reduction_events": {"median": round(kern_ms, 4), "min": round(min(ev_ms), 4)},
        "device_status": bbm.bb_status_str(status),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 5), "traffic": None,
                     "kernel": "cycle kernel launches of one reduction (pack/extract included)"},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(band, w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
