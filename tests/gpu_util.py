"""Helpers for the GPU parity tests: run the HIP path through the C ABI."""
from __future__ import annotations

import os
import sys

import numpy as np

import band_bidiagonal_bulge_amd as bbm


def log(msg: str) -> None:
    """Names the case before each GPU step (flushed, so a fault still shows it)."""
    sys.stdout.write("[gpu] " + msg + "\n")
    sys.stdout.flush()
    sys.stderr.flush()


def gpu_reduce(band: np.ndarray, bw: int, tw: int, tun=None, return_band: bool = False, reps: int = 1):
    import torch
    dev = torch.device("cuda:0")
    tb = torch.from_numpy(np.ascontiguousarray(band)).to(dev)
    n = band.shape[0]
    work = bbm.workspace(n, bw, tw, tb.dtype, dev)
    for _ in range(reps):
        d, e = bbm.reduce(tb, bw, tw, tun, work)
    torch.cuda.synchronize()
    out = [d.cpu().numpy(), e.cpu().numpy()]
    if return_band:
        W, sub = bbm.export_band(work, n, bw, tw, tb.dtype)
        torch.cuda.synchronize()
        out += [W.cpu().numpy(), sub]
    st = bbm.bb_device_status(work.data_ptr(), n, bw, tw, bbm.dtype_code(tb.dtype),
                              torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, bbm.bb_status_str(st)
    return tuple(out)


def weyl_sv_bound(d1, e1, d2, e2) -> float:
    """Upper bound on max_i |sigma_i(B1) - sigma_i(B2)| for upper bidiagonals.

    Singular values of a bidiagonal do not depend on the signs of d, e, and
    by Weyl's inequality they move by at most ||B1 - B2||_2 <= max|dd| + max|de|.
    """
    dd = np.max(np.abs(np.abs(d1.astype(np.float64)) - np.abs(d2.astype(np.float64)))) if d1.size else 0.0
    de = np.max(np.abs(np.abs(e1.astype(np.float64)) - np.abs(e2.astype(np.float64)))) if e1.size else 0.0
    return float(dd + de)


TOL = {"f32": 2e-4, "f64": 1e-10}  # elementwise |d|,|e| and singular values, times ||A||_F
