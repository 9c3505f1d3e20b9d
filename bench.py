#!/usr/bin/env python3
"""Benchmark of the band -> bidiagonal reduction on one MI355X.

One step = one full reduction (pack, every pass, extract) of the workload's
band, already resident in device memory when the timed region starts.

Prints one JSON line:
  metric / unit   effective GB/s = algorithmic bytes of the reduction / time
                  (ms per reduction is ms_per_step)
  roofline        the dominant kernel's algorithmic bytes per launch over its
                  average launch duration (HIP events on the stream the
                  kernels run on), against the published HBM3E peak;
                  working_set names the level that holds the working band
                  (by its size) with that level's datasheet peak and the
                  library's stream (z = x + y) and transpose-add probes over
                  the band's footprint and over 64 MiB, each with its
                  fraction
  ms_per_reduction_events  median and min of the per-step event times
  schedulers_ms   the same path under the step scheduler (the page's one
                  launch per step), the grid-barrier scheduler (the same
                  steps in one launch per pass, a device-wide barrier
                  between steps) and the persistent scheduler, and the sum
                  of the per-pass times below (the group kernel, one launch
                  per pass)
  passes          each pass in a launch of its own (bb_run_pass), timed after
                  the steps; launch_of_pass: which cycle-kernel launch runs
                  each pass in a step
  cpu_baseline    the CPU oracle (one thread) timed on a bounded prefix of the
                  same reduction, in the same unit: median of three samples
  svals           the step after the path: singular values of the workload's
                  bidiagonal by bisection on the GPU (bb_svals), its ALU
                  roofline in Sturm pivots per second, and the bisection
                  oracle timed on a sample of the values
  sym             the symmetric band -> tridiagonal reduction (bb_sym_reduce)
                  on the headline shape and on the page's n = 4096, b = 32
                  one-pass shape: ms, effective GB/s, its cycle kernel's
                  roofline, and the symmetric oracle on the smaller shape
  f16             the same reduction of the headline band in half precision:
                  ms and effective GB/s
  cpu_threaded    the oracle's cycles with each pass's sweeps on all host
                  cores (at most 16), on the whole reduction when it fits the
                  time bound, else on its first pass

--pass-ranges prints the ms of each pass alone, of each consecutive pair of
passes in one launch and of all passes (what sharing a launch gains at each
pass boundary) instead of the bench line.

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


def cpu_baseline(band, w, seconds, samples=3):
    """The oracle (one thread) on a bounded prefix of the reduction: the
    prefix is sized to about seconds / samples of work, run `samples` times,
    and the median rate is the value."""
    import oracle
    oracle.build()
    esize = 8 if w.dtype == "f64" else 4
    # calibrate on a short prefix, then size the sample to about `seconds`
    t0 = time.perf_counter()
    _, _, done = oracle.reduce(band, w.bw, w.tw, max_cycles=100000)
    dt = time.perf_counter() - t0
    rate = alg_bytes_prefix(w.n, w.bw, w.tw, esize, done) / max(dt, 1e-9)
    target = rate * seconds / samples
    # grow the cycle count until the prefix holds about `target` bytes
    lo, hi = done, done
    while alg_bytes_prefix(w.n, w.bw, w.tw, esize, hi) < target and hi < 10 ** 9:
        lo, hi = hi, hi * 2
    for _ in range(12):
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if alg_bytes_prefix(w.n, w.bw, w.tw, esize, mid) < target else (lo, mid)
    ncyc = hi
    rates, times = [], []
    for _ in range(samples):
        t0 = time.perf_counter()
        _, _, done = oracle.reduce(band, w.bw, w.tw, max_cycles=ncyc)
        dt = time.perf_counter() - t0
        nbytes = alg_bytes_prefix(w.n, w.bw, w.tw, esize, done)
        rates.append(nbytes / dt / 1e9)
        times.append(dt)
    return {"value": statistics.median(rates), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of the reduction's cycles in sequential order "
                      f"({nbytes / 1e9:.2f} GB algorithmic), median of {samples} runs "
                      f"({', '.join(f'{t:.1f}' for t in times)} s, one thread)",
            "samples_GBps": [round(r, 3) for r in rates],
            "host": f"{host_model()}, {os.cpu_count()} logical CPUs"}


# The method's arithmetic per pivot of a Sturm count on the Golub-Kahan
# tridiagonal (squares of the off-diagonal formed once per value, outside the
# count): one division, one subtraction and one sign test.  Peak = the chip's
# vector lane-instruction rate for the dtype (fp32 157.3 TFLOP/s, fp64 78.6
# TFLOP/s, two flops per FMA lane-instruction) over those 3 operations, as if
# each were one instruction.  ISSUED_OPS is what the kernel issues per pivot
# (a correctly rounded division takes 10 fp32 / 11 fp64 instructions, the
# pivmin guard 2 / 3, the count 2): its fraction is the issue efficiency.
METHOD_PIVOT_OPS = 3
ISSUED_PIVOT_OPS = {"f32": 15, "f64": 17}
LANE_OPS_PER_S = {"f32": 157.3e12 / 2, "f64": 78.6e12 / 2}


def measure_svals(bbm, torch, d, e, w, steps, stream, cpu_seconds, with_cpu):
    dev = d.device
    dt = bbm.dtype_code(d.dtype)
    n = w.n
    halvings = 26 if w.dtype == "f32" else 55
    work = torch.empty(bbm.bb_svals_workspace_bytes(n, dt), dtype=torch.uint8, device=dev)
    sig = torch.empty(n, dtype=d.dtype, device=dev)
    tree, levels = bbm.bb_svals_split(n, dt)
    sp = stream.cuda_stream

    def run():
        bbm.bb_svals(d.data_ptr(), e.data_ptr(), n, dt, 0, n, 0, 0, sig.data_ptr(), work.data_ptr(), work.numel(),
                     sp)

    run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in evs)
    # the method's work: every value bisected on its own, `halvings` counts
    # of 2n pivots each
    pivots = float(n) * halvings * 2 * n
    rate = pivots / (ms * 1e-3) / 1e9
    peak = LANE_OPS_PER_S[w.dtype] / METHOD_PIVOT_OPS / 1e9
    issue_peak = LANE_OPS_PER_S[w.dtype] / ISSUED_PIVOT_OPS[w.dtype] / 1e9
    out = {"kernel": "k_gk_prep + k_tree + k_bisect", "ms": round(ms, 4), "values": n,
           "split": {"tree_levels": tree, "levels": levels}, "halvings": halvings,
           "roofline": {"bound": "alu", "achieved": round(rate, 2), "peak": round(peak, 1), "unit": "Gpivot/s",
                        "frac": round(rate / peak, 4),
                        "peak_basis": "3 method operations per pivot (division, subtraction, sign test)",
                        "issue_peak": round(issue_peak, 1), "issue_frac": round(rate / issue_peak, 4)}}
    if with_cpu:
        import oracle
        oracle.build_svals()
        dh, eh = d.cpu().numpy(), e.cpu().numpy()
        t0 = time.perf_counter()
        oracle.svals(dh, eh, 0, 8)
        per_value = (time.perf_counter() - t0) / 8
        m = int(max(8, min(n, cpu_seconds / max(per_value, 1e-9))))
        t0 = time.perf_counter()
        oracle.svals(dh, eh, 0, m)
        dtc = time.perf_counter() - t0
        out["cpu_oracle"] = {"value": round(m * halvings * 2.0 * n / dtc / 1e9, 4), "unit": "Gpivot/s", "cores": 1,
                             "kind": "oracle", "sample": f"the {m} largest of {n} values ({dtc:.1f} s, one thread)"}
    return out


def sym_pass_bytes(n, b, t, esize):
    """Algorithmic bytes of one symmetric pass: every cycle reads and writes
    the pivot row segment, the row segments above the block, the block's
    upper triangle and the column segments to its right, once each."""
    bp = b - t
    R = np.arange(max(n - bp - 1, 0), dtype=np.int64)
    K = (n - 2 - R - bp) // b + 1
    Rr = np.repeat(R, K)
    k = np.arange(Rr.size, dtype=np.int64) - np.repeat(np.cumsum(K) - K, K)
    c = Rr + bp + k * b
    ch = np.minimum(c + t, n - 1)
    m = ch - c + 1
    p = np.where(k == 0, Rr, c - b)
    nr = c - p - 1
    nc = np.minimum(ch + b, n - 1) - ch
    return float(np.sum(2.0 * esize * (m + nr * m + m * (m + 1) / 2 + nc * m)))


SYM_SHAPES = [(16384, 64, 16, "f32"), (4096, 32, 31, "f32")]


def measure_sym(bbm, torch, steps, stream, with_cpu):
    out = []
    dev = torch.device("cuda:0")
    for (n, bw, tw, dt) in SYM_SHAPES:
        band_np = bb_inputs.make_band(n, bw, dt, "normal", seed=0)
        band = torch.from_numpy(band_np).to(dev)
        work = bbm.sym_workspace(n, bw, tw, band.dtype, dev)
        esize = 8 if dt == "f64" else 4
        passes = pass_list(bw, tw)
        pbytes = [sym_pass_bytes(n, b, t, esize) for (b, t) in passes]
        bbm.sym_reduce(band, bw, tw, None, work)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            bbm.sym_reduce(band, bw, tw, None, work)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        status = bbm.bb_sym_device_status(work.data_ptr(), n, bw, tw, bbm.dtype_code(band.dtype),
                                          stream.cuda_stream)
        total = sum(pbytes)
        gbps = total / (ms * 1e-3) / 1e9
        entry = {"workload": f"sym-n{n}-bw{bw}-tw{tw}-{dt}-normal", "ms": round(ms, 3), "GBps": round(gbps, 2),
                 "alg_bytes": total, "passes": len(passes), "device_status": bbm.bb_status_str(status),
                 "kernel": "symmetric cycle kernel (k_group with the symmetric half-cycles where the pass's LDS "
                           "ring fits, consecutive such passes in one launch; else k_sym_persist)",
                 "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(gbps / HBM_PEAK_GBPS, 5),
                              "note": "whole reduction over its wall time (the launches are back to back)"}}
        if with_cpu and n <= 4096:
            import oracle
            oracle.build_sym()
            t0 = time.perf_counter()
            oracle.sym_reduce(band_np, bw, tw)
            dtc = time.perf_counter() - t0
            entry["cpu_oracle"] = {"value": round(total / dtc / 1e9, 3), "unit": "GB/s", "cores": 1,
                                   "kind": "oracle", "sample": f"the whole reduction ({dtc:.2f} s, one thread)"}
        out.append(entry)
    return out


def measure_f16(bbm, torch, w, steps, stream):
    """The headline band reduced in half precision (fp16 storage and
    arithmetic, the default scheduler)."""
    band = torch.from_numpy(bb_inputs.make_band(w.n, w.bw, "f16", w.dist, w.seed)).to("cuda:0")
    work = bbm.workspace(w.n, w.bw, w.tw, band.dtype, band.device)
    info = bbm.bb_plan(w.n, w.bw, w.tw, bbm.BB_F16)
    bbm.reduce(band, w.bw, w.tw, None, work)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        bbm.reduce(band, w.bw, w.tw, None, work)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    status = bbm.bb_device_status(work.data_ptr(), w.n, w.bw, w.tw, bbm.BB_F16, stream.cuda_stream)
    gbps = info.alg_bytes / (ms * 1e-3) / 1e9
    return {"workload": f"n{w.n}-bw{w.bw}-tw{w.tw}-f16-{w.dist}", "ms": round(ms, 3), "GBps": round(gbps, 2),
            "alg_bytes": info.alg_bytes, "kernel": "k_group<_Float16> where the pass's LDS ring fits "
                                                 "(consecutive such passes in one launch), else "
                                                 "k_persist<_Float16>",
            "device_status": bbm.bb_status_str(status),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 5),
                         "note": "whole reduction over its wall time (the launches are back to back)"}}


def accuracy_study(n, bw, tw, instances, out_md):
    """Relative singular-value error ||sigma - Sigma|| / ||Sigma|| of the GPU
    reduction in fp64, fp32 and fp16 on bands with known singular values
    (fp64 first stage, fp64 bisection afterwards): the study of the page
    "Accelerating Bidiagonalization of Banded Matrices through Memory-Aware
    Bulge-Chasing on GPUs" (known-spectrum accuracy passage)."""
    import torch
    import band_bidiagonal_bulge_amd as bbm
    dev = torch.device("cuda:0")
    rows = []
    for spectrum in bb_inputs.SPECTRA:
        for seed in range(instances):
            band64, sigma = bb_inputs.known_spectrum_band(n, bw, spectrum, seed=seed)
            for dt in ("f64", "f32", "f16"):
                tb = torch.from_numpy(band64.astype(bb_inputs.np_dtype(dt))).to(dev)
                d, e = bbm.reduce(tb, bw, tw)
                sv = bbm.svals(d.double(), e.double()).cpu().numpy()
                rows.append((spectrum, seed, dt, float(np.linalg.norm(sv - sigma) / np.linalg.norm(sigma))))
    summary = {}
    for dt in ("f64", "f32", "f16"):
        errs = sorted(r[3] for r in rows if r[2] == dt)
        summary[dt] = {"min": errs[0], "median": float(np.median(errs)), "max": errs[-1]}
        for sp in bb_inputs.SPECTRA:
            summary[dt][sp + "_median"] = float(np.median([r[3] for r in rows if r[2] == dt and r[0] == sp]))
    lines = [f"# Accuracy study: n = {n}, BW = {bw}, TW = {tw}, {instances} instances per spectrum", "",
             "Command (repo root, MI355X): `python bench.py --accuracy-study "
             f"--study-n {n} --study-bw {bw} --study-tw {tw} --study-instances {instances}`", "",
             "Relative error ||sigma - Sigma||_2 / ||Sigma||_2 of the singular values after the GPU reduction in",
             "each precision (fp64 first stage, fp64 bisection of the bidiagonal):", "",
             "| precision | min | median | max | arithmetic (median) | logarithmic (median) | quarter-circle (median) |",
             "|---|---|---|---|---|---|---|"]
    for dt, v in summary.items():
        lines.append(f"| {dt} | {v['min']:.2e} | {v['median']:.2e} | {v['max']:.2e} | {v['arithmetic_median']:.2e} | "
                     f"{v['logarithmic_median']:.2e} | {v['quarter_circle_median']:.2e} |")
    lines += ["", "Every instance:", "", "| spectrum | seed | precision | relative error |", "|---|---|---|---|"]
    lines += [f"| {sp} | {sd} | {dt} | {er:.3e} |" for (sp, sd, dt, er) in rows]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps({"accuracy_study": {"n": n, "bw": bw, "tw": tw, "instances_per_spectrum": instances,
                                         "summary": summary}}), flush=True)


def host_model() -> str:
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    """Host threads for the threaded CPU chaser: the cores this process may
    run on, at most 16 (the host share that goes with one GPU).  The chaser
    caps them further per pass as the page does (2n/(3b), n/256)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_threaded(band, w, seconds):
    import oracle
    oracle.build_mt()
    esize = 8 if w.dtype == "f64" else 4
    passes = pass_list(w.bw, w.tw)
    cyc = []
    for (b, t) in passes:
        R = np.arange(max(w.n - (b - t) - 1, 0), dtype=np.int64)
        cyc.append(int(np.sum((w.n - 2 - R - (b - t)) // b + 1)))
    threads = host_cores()
    t0 = time.perf_counter()
    _, _, used = oracle.reduce_mt(band, w.bw, w.tw, threads=-threads, max_passes=1)
    dt = time.perf_counter() - t0
    npass = 1
    if dt * len(passes) < seconds and len(passes) > 1:
        t0 = time.perf_counter()
        _, _, used = oracle.reduce_mt(band, w.bw, w.tw, threads=-threads)
        dt = time.perf_counter() - t0
        npass = len(passes)
    nbytes = alg_bytes_prefix(w.n, w.bw, w.tw, esize, sum(cyc[:npass]))
    what = "the whole reduction" if npass == len(passes) else "its first pass"
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": used, "kind": "oracle-threaded",
            "sample": f"{what} ({npass} of {len(passes)} passes, {nbytes / 1e9:.2f} GB algorithmic, "
                      f"{dt:.2f} s, sweeps of a pass on {used} threads)"}


def kernel_source_hash() -> str:
    """Hash of the sources of the reduction's kernels and their launch set-up
    (every HIP source but the singular-value step's, the symmetric
    reduction's and the bandwidth probes'): stored counter readings
    are only valid for it."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "band_bidiagonal_bulge_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.startswith("bb_svals") or f.startswith("bb_sym") or f.startswith("bb_probe"):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per cycle-kernel launch from the stored counter readings
    (profiles/traffic_<workload>.json, written by --ingest-counters), or None
    when they are missing or were taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t


# Published peak of the 256 MiB Infinity Cache of the CDNA 3 part (MI300X,
# 17.2 TB/s); MI355X keeps the same 256 MiB last-level cache in front of HBM.
# Used as the datasheet figure for the level that holds a working band.
IC_PEAK_GBPS = 17200.0
L2_PER_XCD = 4 << 20
IC_BYTES = 256 << 20


def memory_level(nbytes: int) -> str:
    """The level whose capacity bounds a working set that every XCD touches
    through agent-coherent accesses: one XCD's L2 cannot hold a set above 4
    MiB, the Infinity Cache holds up to 256 MiB, HBM the rest."""
    if nbytes <= L2_PER_XCD:
        return "l2"
    return "infinity_cache" if nbytes <= IC_BYTES else "hbm"


def probe_ceilings(bbm, torch, dev, stream, sizes, reps=5, launch_bytes=4e9):
    """Measured ceilings of the level that holds the working band, from the
    library's two probes (bb_probe_stream: z = x + y; bb_probe_transpose_add:
    B = A + A^T), each over a footprint of every size in `sizes` bytes (all
    operands together), repeated inside one launch until the launch moves
    about `launch_bytes` (each repetition on other XCDs), timed with events on
    the stream it runs on, best of `reps` launches.  12 bytes move per
    element and repetition."""
    sp = stream.cuda_stream
    out = []

    def timed(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            best = min(best, a.elapsed_time(b))
        return round(nbytes / (best * 1e-3) / 1e9, 1), round(best * 1e3, 1)

    for size in sizes:
        n = max(4, (size // 12) // 4 * 4)
        r = max(1, int(launch_bytes // (12 * n)))
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.ones(n, dtype=torch.float32, device=dev)
        z = torch.zeros(n, dtype=torch.float32, device=dev)
        gbps, us = timed(lambda: bbm.bb_probe_stream(x.data_ptr(), y.data_ptr(), z.data_ptr(), n, r, sp), 12 * n * r)
        out.append({"probe": "stream z = x + y", "footprint_mib": round(12 * n / 2**20, 2), "repetitions": r,
                    "GBps": gbps, "us_per_launch": us})
        del x, y, z
        m = max(1, int((size // 8) ** 0.5))
        r = max(1, int(launch_bytes // (12 * m * m)))
        a = torch.ones(m, m, dtype=torch.float32, device=dev)
        b = torch.zeros(m, m, dtype=torch.float32, device=dev)
        gbps, us = timed(lambda: bbm.bb_probe_transpose_add(a.data_ptr(), b.data_ptr(), m, r, sp), 12 * m * m * r)
        out.append({"probe": f"transpose-add B = A + A^T, m = {m}", "footprint_mib": round(8 * m * m / 2**20, 2),
                    "repetitions": r, "GBps": gbps, "us_per_launch": us})
        del a, b
    return out


def norm_clocks(bbm, torch, dev, stream, reps=20000):
    """Shader clocks per reflector norm in one wave (bb_probe_norm_clocks):
    the serial FMA chain the reduction uses against a DPP cross-lane
    reduction, for the register tiles of 17 and 33 entries."""
    x = torch.rand(64, dtype=torch.float32, device=dev)
    out = torch.empty(64, dtype=torch.float32, device=dev)
    clk = torch.zeros(1, dtype=torch.int64, device=dev)
    res = {}
    for m in (17, 33):
        for mode, name in ((0, "serial_fma"), (1, "dpp_reduction")):
            best = None
            for _ in range(3):
                bbm.bb_probe_norm_clocks(m, mode, reps, x.data_ptr(), out.data_ptr(), clk.data_ptr(), stream.cuda_stream)
                torch.cuda.synchronize()
                c = clk.item() / reps
                best = c if best is None else min(best, c)
            res[f"m{m}_{name}"] = round(best, 1)
    return res


def scheduler_times(bbm, torch, tb, w, dt, work, stream, reps=2):
    """Median ms per reduction of the whole path under the step scheduler
    (one launch per step, the page's design), the grid-barrier scheduler and
    the persistent scheduler, for comparison with the default."""
    out = {}
    for name, code in (("step", bbm.BB_SCHED_STEP), ("barrier", bbm.BB_SCHED_BARRIER),
                       ("persistent", bbm.BB_SCHED_PERSISTENT)):
        tun = bbm.tuning(scheduler=code)
        bbm.reduce(tb, w.bw, w.tw, tun, work)
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            bbm.reduce(tb, w.bw, w.tw, tun, work)
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        out[name] = round(statistics.median(ms), 3)
    return out


def pass_ranges(bbm, torch, tb, w, dt, info, wp, wn, stream, reps=3):
    """Median ms of ranges of passes run by one bb_run_passes call under the
    default scheduler (consecutive group-kernel passes share a launch): each
    pass alone, each pair of consecutive passes, and all of them.  The
    passes before a range run untimed first, so each range starts from the
    working band it would see in a reduction."""
    sp = stream.cuda_stream
    one_each = bbm.tuning(scheduler=bbm.BB_SCHED_GROUP)
    ranges = [(p, 1) for p in range(info.passes)] + [(p, 2) for p in range(info.passes - 1)] + [(0, info.passes)]
    out = []
    for (first, count) in ranges:
        ms = []
        for _ in range(reps):
            bbm.bb_pack(tb.data_ptr(), tb.stride(0), w.n, w.bw, w.tw, dt, wp, wn, sp)
            if first:
                bbm.bb_run_passes(w.n, w.bw, w.tw, dt, 0, first, wp, wn, None, sp)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            bbm.bb_run_passes(w.n, w.bw, w.tw, dt, first, count, wp, wn, None if count > 1 else one_each, sp)
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        out.append({"first": first, "count": count, "ms": round(statistics.median(ms), 3)})
    return out


def pass_tables(w):
    """Per pass: (b, t, algorithmic bytes) of the workload."""
    esize = 8 if w.dtype == "f64" else 4
    out = []
    for (b, t) in pass_list(w.bw, w.tw):
        bp = b - t
        R = np.arange(max(w.n - bp - 1, 0), dtype=np.int64)
        K = (w.n - 2 - R - bp) // b + 1
        Rr = np.repeat(R, K)
        k = np.arange(Rr.size, dtype=np.int64) - np.repeat(np.cumsum(K) - K, K)
        c = Rr + bp + k * b
        ch = np.minimum(c + t, w.n - 1)
        r = np.where(k == 0, Rr, c - b)
        m = ch - c + 1
        cols = np.minimum(c + t + b, w.n - 1) - c + 1
        out.append((b, t, float(np.sum(2.0 * m * ((ch - r + 1) + cols - m) * esize))))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=bb_inputs.HEADLINE)
    ap.add_argument("--scheduler", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-svals", action="store_true")
    ap.add_argument("--no-sym", action="store_true")
    ap.add_argument("--no-f16", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the bandwidth probes of the working set's level")
    ap.add_argument("--no-schedulers", action="store_true", help="skip the step / persistent scheduler times")
    ap.add_argument("--pass-ranges", action="store_true",
                    help="time each pass alone, each consecutive pair in one launch and all passes, then exit")
    ap.add_argument("--no-per-pass", action="store_true",
                    help="skip the per-pass breakdown (each pass in a launch of its own, after the steps)")
    ap.add_argument("--accuracy-study", action="store_true",
                    help="run the known-spectrum accuracy study instead of the bench (writes --study-out)")
    ap.add_argument("--study-n", type=int, default=512)
    ap.add_argument("--study-bw", type=int, default=32)
    ap.add_argument("--study-tw", type=int, default=16)
    ap.add_argument("--study-instances", type=int, default=10)
    ap.add_argument("--study-out", default=os.path.join("gpurun_out", "accuracy_study.md"))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc runs (no GPU)")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args.workload, *args.ingest_counters, args.copy_probe_mib)
        return
    if args.accuracy_study:
        os.makedirs(os.path.dirname(os.path.abspath(args.study_out)), exist_ok=True)
        accuracy_study(args.study_n, args.study_bw, args.study_tw, args.study_instances, args.study_out)
        return
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
    passes = pass_tables(w)
    assert len(passes) == info.passes
    work = bbm.workspace(w.n, w.bw, w.tw, tb.dtype, dev)
    d = torch.empty(w.n, dtype=tb.dtype, device=dev)
    e = torch.empty(w.n - 1, dtype=tb.dtype, device=dev)
    tun = bbm.tuning(scheduler=args.scheduler)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    wp, wn = work.data_ptr(), work.numel()

    # the cycle-kernel launches of one reduction: under the default scheduler
    # consecutive passes on the group kernel share one launch
    launch_of = bbm.bb_launch_plan(w.n, w.bw, w.tw, dt, tun)
    nlaunch = len(set(x for x in launch_of if x >= 0))

    def one(rev=None, sev=None):
        # pack, every pass (one bb_run_passes call, as bb_reduce makes it),
        # extract; events on the stream the kernels run on bracket the passes
        # and the whole step
        if sev is not None:
            sev[0].record(stream)
        bbm.bb_pack(tb.data_ptr(), tb.stride(0), w.n, w.bw, w.tw, dt, wp, wn, sp)
        if rev is not None:
            rev[0].record(stream)
        bbm.bb_run_passes(w.n, w.bw, w.tw, dt, 0, info.passes, wp, wn, tun, sp)
        if rev is not None:
            rev[1].record(stream)
        bbm.bb_extract(wp, wn, w.n, w.bw, w.tw, dt, d.data_ptr(), e.data_ptr(), sp)
        if sev is not None:
            sev[1].record(stream)

    def per_pass(reps=3):
        """Each pass in a launch of its own (bb_run_pass): median ms per pass."""
        ms = [[] for _ in range(info.passes)]
        for _ in range(reps):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(info.passes)]
            bbm.bb_pack(tb.data_ptr(), tb.stride(0), w.n, w.bw, w.tw, dt, wp, wn, sp)
            for p in range(info.passes):
                evs[p][0].record(stream)
                bbm.bb_run_pass(w.n, w.bw, w.tw, dt, p, wp, wn, tun, sp)
                evs[p][1].record(stream)
            torch.cuda.synchronize()
            for p in range(info.passes):
                ms[p].append(evs[p][0].elapsed_time(evs[p][1]))
        return [statistics.median(x) for x in ms]

    if args.pass_ranges:
        print(json.dumps({"workload": w.name, "pass_ranges": pass_ranges(bbm, torch, tb, w, dt, info, wp, wn, stream)}),
              flush=True)
        return

    if args.copy_probe_mib:
        nb = args.copy_probe_mib << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one(rev[s], sev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    status = bbm.bb_device_status(wp, w.n, w.bw, w.tw, dt, sp)
    run_ms = [a.elapsed_time(b) for (a, b) in rev]
    step_ms = [a.elapsed_time(b) for (a, b) in sev]
    ms_per_step = wall * 1e3 / args.steps
    value = info.alg_bytes / (ms_per_step * 1e-3) / 1e9
    # dominant kernel: the cycle kernel; algorithmic bytes per launch over the
    # average launch duration (the passes' event time over the launches)
    launches = nlaunch * args.steps
    avg_launch_ms = sum(run_ms) / launches
    bytes_per_launch = sum(p[2] for p in passes) / nlaunch
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    pass_ms = None if args.no_per_pass else per_pass()
    traffic = stored_traffic(w.name)

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
        "device_status": bbm.bb_status_str(status),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 5),
                     "traffic": None if traffic is None else round(traffic["hbm_bytes_per_launch"], 1),
                     "kernel": "cycle kernel (k_group where the pass's LDS ring fits, consecutive such passes "
                               "in one launch, fp32 passes with t = 31 or 32 on windows of the rows; else "
                               "k_persist, one launch per pass)",
                     "launches": launches, "avg_launch_ms": round(avg_launch_ms, 4),
                     "alg_bytes_per_launch": bytes_per_launch},
        "ms_per_reduction_events": {"median": round(statistics.median(step_ms), 4), "min": round(min(step_ms), 4)},
        "launch_of_pass": launch_of,
        # each pass in a launch of its own, timed after the steps
        "passes": [{"b": b, "t": t, "alg_bytes": ab} if pass_ms is None else
                   {"b": b, "t": t, "alg_bytes": ab, "median_ms": round(pass_ms[i], 4),
                    "GBps": round(ab / (pass_ms[i] * 1e-3) / 1e9, 2)}
                   for i, (b, t, ab) in enumerate(passes)],
    }
    ws = int(work.numel())
    level = {"working_set_bytes": ws, "level": memory_level(ws)}
    if level["level"] == "infinity_cache":
        level.update({"datasheet_peak": IC_PEAK_GBPS, "datasheet_frac": round(achieved / IC_PEAK_GBPS, 5),
                      "datasheet": "MI300X Infinity Cache peak (the CDNA 3 part's published figure)"})
    if not args.no_ceiling:
        probes = probe_ceilings(bbm, torch, dev, stream, [ws, 64 << 20])
        for p in probes:
            p["frac"] = round(achieved / p["GBps"], 5)
        level["probes"] = probes
        out["norm_clocks"] = norm_clocks(bbm, torch, dev, stream)
    out["roofline"]["working_set"] = level
    if not args.no_schedulers:
        out["schedulers_ms"] = scheduler_times(bbm, torch, tb, w, dt, work, stream)
        out["schedulers_ms"]["default"] = round(statistics.median(step_ms), 3)
        if pass_ms is not None:
            out["schedulers_ms"]["group_per_pass"] = round(sum(pass_ms), 3)
    if not args.no_svals:
        out["svals"] = measure_svals(bbm, torch, d, e, w, args.steps, stream, args.cpu_seconds / 3, not args.no_cpu)
    if not args.no_f16:
        out["f16"] = measure_f16(bbm, torch, w, max(1, min(args.steps, 3)), stream)
    if not args.no_sym:
        out["sym"] = measure_sym(bbm, torch, max(1, min(args.steps, 3)), stream, not args.no_cpu)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(band, w, args.cpu_seconds)
        out["cpu_threaded"] = cpu_threaded(band, w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def _read_counter_csv(path, counter):
    """Per-dispatch rows of a rocprofv3 --pmc counter_collection.csv:
    [(kernel_name, value)] in dispatch order."""
    import csv
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r.get("Counter_Name") == counter:
                rows.append((int(r.get("Dispatch_Id", 0)), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(k, v) for (_, k, v) in rows]


def is_cycle_kernel(name, dtype):
    """The workload's cycle kernel in a profiler row: the general band's
    k_group / k_persist / k_step / k_barrier in the workload's element type
    (not the symmetric sweep groups, not the half-precision run)."""
    ctype = {"f32": "float", "f64": "double", "f16": "_Float16"}[dtype]
    if "k_group<" + ctype + "," in name:  # k_group<T, MAXM, SC, SYM>: not the symmetric one
        return not name.split("k_group<", 1)[1].split(">", 1)[0].endswith("true")
    return any(k + ctype + "," in name for k in ("k_persist<", "k_step<", "k_barrier<"))


def ingest_counters(workload, fetch_csv, write_csv, copy_mib):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the cycle kernels, each
    scaled by what the same counter reads for the plain copy of copy_mib MiB
    (which moves exactly copy_mib MiB each way)."""
    if copy_mib <= 0:
        raise SystemExit("--copy-probe-mib is needed to scale the counters")
    w = bb_inputs.WORKLOADS[workload]
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(), "copy_probe_mib": copy_mib}
    total = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _read_counter_csv(path, name)
        copy = [v for (k, v) in rows if "copybuffer" in k.lower()]
        cyc = [v for (k, v) in rows if is_cycle_kernel(k, w.dtype)]
        if not copy or not cyc:
            raise SystemExit(f"{path}: no copy-probe or cycle-kernel rows for {name}")
        factor = (copy_mib * 1024.0) / max(copy)  # KiB the copy moves / KiB counted
        per_launch = sum(cyc) / len(cyc) * 1024.0 * factor
        out[name] = {"copy_probe_kib": max(copy), "scale": factor, "cycle_kernel_kib_mean": sum(cyc) / len(cyc),
                     "launches": len(cyc), "bytes_per_launch": per_launch}
        total += per_launch
    out["hbm_bytes_per_launch"] = total
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(path)


if __name__ == "__main__":
    main()
