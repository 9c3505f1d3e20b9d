"""The fp32 noise floor of the reduction: how far two correct fp32 results of
the same band may lie apart, measured as the distance between the oracle in
fp32 and the same oracle in fp64 on the fp32-rounded input (the fp64 run is the
accuracy reference).  Prints, per workload and seed, relative to ||A||_F:

  elementwise  max over i of | |d32_i| - |d64_i| | and of the same for e
  sv           max over i of |sigma32_i - sigma64_i|, singular values of the
               two bidiagonals (fp64 Golub-Kahan eigenvalues)

Stored outputs (``<workload>.npz`` with d64/e64, written by make_golden.py
--f64ref) are read; other (workload, seed) pairs are computed here with the
threaded oracle runner (bitwise equal to the sequential oracle).  Calls only
``oracle/`` and ``bb_inputs``.

Usage:  python tests/golden/noise_floor.py [WORKLOAD:SEED ...]
        (default: the stored fp32 outputs, n = 4096 seeds 0-2, n = 16384 seeds 1-2)
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, HERE)

import bb_inputs  # noqa: E402
import oracle  # noqa: E402
from make_golden import bidiag_singular_values  # noqa: E402

DEFAULT = ["n4096-bw32-tw16-f32-normal:1", "n4096-bw32-tw16-f32-normal:2",
           "n16384-bw64-tw16-f32-normal:1", "n16384-bw64-tw16-f32-normal:2"]


def floors(d32, e32, d64, e64, sv32, sv64, fro):
    el = max(np.max(np.abs(np.abs(d32.astype(np.float64)) - np.abs(d64))),
             np.max(np.abs(np.abs(e32.astype(np.float64)) - np.abs(e64))) if e64.size else 0.0)
    return el / fro, float(np.max(np.abs(sv32 - sv64))) / fro


def stored():
    out = []
    for f in sorted(os.listdir(HERE)):
        if not f.endswith(".npz") or f.startswith("sym-"):
            continue
        z = np.load(os.path.join(HERE, f))
        if "d64" not in z.files:
            continue
        w = bb_inputs.WORKLOADS[f[:-4]]
        out.append((w.name, w.seed, "stored") + floors(z["d"], z["e"], z["d64"], z["e64"], z["sv"], z["sv64"],
                                                       float(z["fro"])))
    return out


def computed(name, seed):
    w = bb_inputs.WORKLOADS[name]
    band = bb_inputs.make_band(w.n, w.bw, w.dtype, w.dist, seed=seed)
    fro = float(np.sqrt(np.sum(band.astype(np.float64) ** 2)))
    d32, e32, _ = oracle.reduce_mt(band, w.bw, w.tw, threads=-16)
    d64, e64, _ = oracle.reduce_mt(band, w.bw, w.tw, threads=-16, compute="f64")
    return (name, seed, "computed") + floors(d32, e32, d64, e64, bidiag_singular_values(d32, e32),
                                            bidiag_singular_values(d64, e64), fro)


def main(argv):
    oracle.build_mt()
    rows = stored()
    for item in (argv or DEFAULT):
        name, seed = item.split(":")
        rows.append(computed(name, int(seed)))
    print("| workload | seed | source | elementwise / ‖A‖_F | singular values / ‖A‖_F |")
    print("|---|---|---|---|---|")
    for (name, seed, src, el, sv) in sorted(rows):
        print(f"| {name} | {seed} | {src} | {el:.3e} | {sv:.3e} |", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
