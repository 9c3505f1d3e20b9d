"""Writes the stored oracle outputs used by the full-size parity tests.

Calls only the CPU oracle (``oracle/``) and the seeded input generators
(``bb_inputs``); nothing here touches the HIP library.  For each workload it
stores, in ``<workload>.npz``:

  d, e        the oracle's bidiagonal in the workload's dtype (gate reference)
  sv          singular values of that bidiagonal, descending, computed in fp64
              as the non-negative eigenvalues of the 2n x 2n Golub-Kahan
              tridiagonal (LAPACK sterf through SciPy)
  fro         ||A||_F of the cast input, in fp64
  input_sha   sha256 of the cast input band bytes (detects generator drift)
  oracle_sha  sha256 of the oracle sources the values came from
and, with --f64ref for an fp32 workload, d64/e64/sv64 from the same oracle run
in fp64 on the fp32-rounded input (the accuracy reference and noise floor).

Two more kinds cover the shapes the bench line reports beside the workloads:
  --sym N BW TW   the symmetric band -> tridiagonal oracle on the seeded
                  N(0,1) fp32 band (d, e; eigenvalues in 'ev'), stored as
                  sym-n<N>-bw<BW>-tw<TW>-f32-normal.npz
  --f16 WORKLOAD  the workload's band cast to binary16, reduced by the
                  emulated-binary16 oracle, stored as the workload name with
                  its dtype replaced by f16

Usage:  python tests/golden/make_golden.py [--f64ref] WORKLOAD [WORKLOAD ...]
        python tests/golden/make_golden.py --sym 16384 64 16
        python tests/golden/make_golden.py --f16 n16384-bw64-tw16-f32-normal
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sys
import time

import numpy as np
import scipy.linalg

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import bb_inputs  # noqa: E402
import oracle  # noqa: E402


def bidiag_singular_values(d: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Singular values (descending) of upper bidiagonal (d, e), in fp64."""
    d = np.asarray(d, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    n = d.size
    off = np.zeros(2 * n - 1)
    off[0::2] = d
    off[1::2] = e
    ev = scipy.linalg.eigvalsh_tridiagonal(np.zeros(2 * n), off, lapack_driver="sterf")
    # eigenvalues come in +-sigma pairs: keep the n largest (non-negative)
    return np.sort(ev)[::-1][:n].copy()


def oracle_sha(files=("bb_oracle.c", "bb_oracle_body.h")) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "oracle", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


SYM_FILES = ("bb_oracle_sym.c", "bb_oracle_sym_body.h")
F16_FILES = ("bb_oracle_f16.cpp", "bb_oracle_body.h")


def make_sym(n: int, bw: int, tw: int) -> None:
    oracle.build_sym()
    band = bb_inputs.make_band(n, bw, "f32", "normal", seed=0)
    t0 = time.time()
    d, e = oracle.sym_reduce(band, bw, tw)
    secs = time.time() - t0
    ev = scipy.linalg.eigvalsh_tridiagonal(d.astype(np.float64), e.astype(np.float64), lapack_driver="sterf")
    name = f"sym-n{n}-bw{bw}-tw{tw}-f32-normal"
    np.savez_compressed(os.path.join(HERE, name + ".npz"), d=d, e=e, ev=ev, oracle_seconds=secs,
                        input_sha=hashlib.sha256(band.tobytes()).hexdigest(), oracle_sha=oracle_sha(SYM_FILES))
    print(f"{name}: symmetric oracle {secs:.1f} s", flush=True)


def make_f16(workload: str) -> None:
    oracle.build_f16()
    w = bb_inputs.WORKLOADS[workload]
    band = bb_inputs.make_band(w.n, w.bw, "f16", w.dist, w.seed)
    t0 = time.time()
    d, e = oracle.reduce(band, w.bw, w.tw)
    secs = time.time() - t0
    name = workload.replace("-" + w.dtype + "-", "-f16-")
    np.savez_compressed(os.path.join(HERE, name + ".npz"), d=d, e=e, oracle_seconds=secs,
                        fro=np.linalg.norm(band.astype(np.float64)),
                        input_sha=hashlib.sha256(band.tobytes()).hexdigest(), oracle_sha=oracle_sha(F16_FILES))
    print(f"{name}: binary16 oracle {secs:.1f} s", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="*")
    ap.add_argument("--f64ref", action="store_true")
    ap.add_argument("--sym", nargs=3, type=int, metavar=("N", "BW", "TW"))
    ap.add_argument("--f16", metavar="WORKLOAD")
    ap.add_argument("--resv", action="store_true",
                    help="only recompute sv/sv64 from the stored d, e")
    args = ap.parse_args()
    if args.sym:
        make_sym(*args.sym)
    if args.f16:
        make_f16(args.f16)
    if args.resv:
        for name in args.workloads:
            path = os.path.join(HERE, name + ".npz")
            z = dict(np.load(path))
            z["sv"] = bidiag_singular_values(z["d"], z["e"])
            if "d64" in z:
                z["sv64"] = bidiag_singular_values(z["d64"], z["e64"])
            np.savez_compressed(path, **z)
        return
    oracle.build()
    for name in args.workloads:
        w = bb_inputs.WORKLOADS[name]
        band = bb_inputs.make_workload(w)
        out = dict(
            input_sha=hashlib.sha256(band.tobytes()).hexdigest(),
            oracle_sha=oracle_sha(),
            fro=np.linalg.norm(band.astype(np.float64)),
        )
        t0 = time.time()
        d, e = oracle.reduce(band, w.bw, w.tw)
        out.update(d=d, e=e, oracle_seconds=time.time() - t0)
        out["sv"] = bidiag_singular_values(d, e)
        print(f"{name}: oracle {out['oracle_seconds']:.1f} s", flush=True)
        if args.f64ref and w.dtype == "f32":
            t0 = time.time()
            d64, e64 = oracle.reduce(band, w.bw, w.tw, compute="f64")
            out.update(d64=d64, e64=e64, sv64=bidiag_singular_values(d64, e64))
            print(f"{name}: fp64 oracle {time.time() - t0:.1f} s", flush=True)
        np.savez_compressed(os.path.join(HERE, name + ".npz"), **out)


if __name__ == "__main__":
    main()
