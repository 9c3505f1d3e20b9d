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


def assert_bits_equal(a, b, what: str = "") -> int:
    """Bit patterns equal, except that a zero may differ from the other zero
    in sign (the documented sign-of-zero caveat: a full-width register tile
    over entries known to hold +0 can turn a -0 partial sum into +0).
    Returns how many entries differ only in the sign of a zero."""
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype, (what, a.shape, b.shape, a.dtype, b.dtype)
    ut = {2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize]
    diff = a.view(ut) != b.view(ut)
    zero_sign = diff & (a == 0) & (b == 0)
    bad = diff & ~zero_sign
    assert not bad.any(), f"{what}: {int(bad.sum())} entries differ in their bits, first at {np.argwhere(bad)[:3].tolist()}"
    return int(zero_sign.sum())


TOL = {"f32": 2e-4, "f64": 1e-10}  # elementwise |d|,|e| and singular values, times ||A||_F
