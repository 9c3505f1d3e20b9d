"""Band -> bidiagonal reduction by Householder bulge chasing on MI355X (gfx950).

The reduction runs in the HIP library ``libbb.so`` (C ABI in include/bb.h).
This package is its thin Python binding: the ``bb_*`` functions mirror the C
entry points, and :func:`reduce` wraps them for torch tensors (torch is used
for device memory and the stream only).
"""
from __future__ import annotations

from ._lib import (BB_ERR_TIMEOUT, BB_ERR_WORKSPACE, BB_NOALLOC_SCRATCH_BYTES, BB_F16, BB_F32, BB_F64, BB_OK, BB_SCHED_BARRIER, BB_SCHED_DEFAULT, BB_SCHED_GROUP, BB_SCHED_PERSISTENT, BB_SCHED_STEP, EXPORTS,
                   BBError,
                   bb_device_status, bb_export_band, bb_extract, bb_pack, bb_plan, bb_plan_info, bb_reduce,
                   bb_reduce_noalloc,
                   bb_launch_plan, bb_probe_norm_clocks, bb_probe_stream, bb_probe_transpose_add, bb_run_pass, bb_run_passes,
                   bb_status_str, bb_svals, bb_svals_split, bb_svals_workspace_bytes, bb_sym_device_status,
                   bb_sym_export_band, bb_sym_reduce, bb_sym_workspace_bytes, bb_tuning,
                   bb_workspace_bytes, lib)

__all__ = ["reduce", "export_band", "workspace", "tuning", "dtype_code", "bb_plan", "bb_workspace_bytes",
           "bb_reduce", "bb_reduce_noalloc", "bb_pack", "bb_run_pass", "bb_run_passes", "bb_launch_plan", "bb_extract", "bb_export_band", "bb_device_status", "bb_svals", "bb_svals_workspace_bytes", "bb_svals_split",
           "bb_sym_workspace_bytes", "bb_sym_reduce", "bb_sym_export_band", "bb_sym_device_status",
           "bb_status_str", "svals", "sym_reduce", "sym_workspace", "BBError", "EXPORTS"]


def dtype_code(torch_dtype) -> int:
    import torch
    if torch_dtype == torch.float32:
        return BB_F32
    if torch_dtype == torch.float64:
        return BB_F64
    if torch_dtype == torch.float16:
        return BB_F16
    raise TypeError("band must be float16, float32 or float64")


def tuning(scheduler: int = 0, stagger: int = 0, max_blocks: int = 0, threads_per_block: int = 0,
           spin_limit: int = 0, group_sweeps: int = 0) -> bb_tuning:
    return bb_tuning(scheduler, stagger, max_blocks, threads_per_block, spin_limit, group_sweeps, 0)


def workspace(n: int, bw: int, tw: int, torch_dtype, device="cuda"):
    """Device workspace for bb_reduce as a uint8 tensor."""
    import torch
    nbytes = bb_workspace_bytes(n, bw, tw, dtype_code(torch_dtype))
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _check_workspace(work, device) -> None:
    import torch
    if work.dtype != torch.uint8 or work.dim() != 1 or not work.is_contiguous():
        raise ValueError("work must be a contiguous 1-D uint8 tensor (sizes are in bytes)")
    if work.device != device:
        raise ValueError(f"work is on {work.device}, the band on {device}")


def reduce(band, bw: int, tw: int, tun: bb_tuning | None = None, work=None, stream=None, check: bool = False):
    """Reduces a device band (n, >= bw+1) float16/float32/float64 tensor; returns (d, e).

    Row i of ``band`` holds A(i, i..i+bw).  Runs on ``stream`` (default: the
    current torch stream) asynchronously.  ``work`` may be a preallocated
    workspace from :func:`workspace` (a uint8 tensor on the band's device).
    With ``check``, waits for the stream and raises :class:`BBError` when a
    device-side wait expired (BB_ERR_TIMEOUT): d and e are then not valid.
    """
    import torch
    if not band.is_cuda or band.dim() != 2 or band.stride(1) != 1:
        raise ValueError("band must be a 2-D device tensor with unit column stride")
    n = band.shape[0]
    dt = dtype_code(band.dtype)
    if work is None:
        work = workspace(n, bw, tw, band.dtype, band.device)
    _check_workspace(work, band.device)
    d = torch.empty(n, dtype=band.dtype, device=band.device)
    e = torch.empty(max(n - 1, 0), dtype=band.dtype, device=band.device)
    s = stream if stream is not None else torch.cuda.current_stream(band.device)
    bb_reduce(band.data_ptr(), band.stride(0), n, bw, tw, dt, d.data_ptr(), e.data_ptr() if n > 1 else 0,
              work.data_ptr(), work.numel(), tun, s.cuda_stream)
    if check:
        st = bb_device_status(work.data_ptr(), n, bw, tw, dt, s.cuda_stream)
        if st != BB_OK:
            raise BBError(st, "bb_reduce")
    return d, e


def export_band(work, n: int, bw: int, tw: int, torch_dtype, stream=None):
    """Working band left in ``work`` as an (n, ld) tensor and its sub offset."""
    import torch
    info = bb_plan(n, bw, tw, dtype_code(torch_dtype))
    out = torch.empty((n, info.ld), dtype=torch_dtype, device=work.device)
    s = stream if stream is not None else torch.cuda.current_stream(work.device)
    bb_export_band(work.data_ptr(), n, bw, tw, dtype_code(torch_dtype), out.data_ptr(), s.cuda_stream)
    return out, info.sub


def svals(d, e, i0: int = 0, i1: int | None = None, levels: int = 0, tree_levels: int = 0, work=None,
          stream=None):
    """Singular values i0..i1-1 (descending) of the upper bidiagonal given by
    device tensors d (n) and e (n-1), by bisection on the Golub-Kahan
    tridiagonal; returns a device tensor of i1-i0 values.  tree_levels and
    levels split the work (0: chosen for the size, tree_levels -1: no shared
    tree); they do not change the result."""
    import torch
    if not d.is_cuda or d.dim() != 1 or not d.is_contiguous():
        raise ValueError("d must be a contiguous 1-D device tensor")
    n = d.shape[0]
    if e.dtype != d.dtype or e.numel() != max(n - 1, 0) or (n > 1 and (not e.is_cuda or not e.is_contiguous())):
        raise ValueError("e must be a contiguous device tensor of n-1 entries of d's dtype")
    dt = dtype_code(d.dtype)
    i1 = n if i1 is None else i1
    out = torch.empty(max(i1 - i0, 0), dtype=d.dtype, device=d.device)
    if work is None:
        work = torch.empty(bb_svals_workspace_bytes(n, dt), dtype=torch.uint8, device=d.device)
    s = stream if stream is not None else torch.cuda.current_stream(d.device)
    bb_svals(d.data_ptr(), e.data_ptr() if n > 1 else 0, n, dt, i0, i1, tree_levels, levels,
             out.data_ptr() if out.numel() else 0, work.data_ptr(), work.numel(), s.cuda_stream)
    return out


def sym_workspace(n: int, bw: int, tw: int, torch_dtype, device="cuda"):
    """Device workspace for bb_sym_reduce as a uint8 tensor."""
    import torch
    return torch.empty(bb_sym_workspace_bytes(n, bw, tw, dtype_code(torch_dtype)), dtype=torch.uint8, device=device)


def sym_reduce(band, bw: int, tw: int, tun: bb_tuning | None = None, work=None, stream=None,
               check: bool = False):
    """Symmetric band -> tridiagonal of a device band (n, >= bw+1) float32 or
    float64 tensor, row i holding A(i, i..i+bw); returns (d, e) device
    tensors.  ``work``: a uint8 tensor on the band's device; ``check`` as for
    :func:`reduce`."""
    import torch
    if not band.is_cuda or band.dim() != 2 or band.stride(1) != 1:
        raise ValueError("band must be a 2-D device tensor with unit column stride")
    n = band.shape[0]
    dt = dtype_code(band.dtype)
    if work is None:
        work = sym_workspace(n, bw, tw, band.dtype, band.device)
    _check_workspace(work, band.device)
    d = torch.empty(n, dtype=band.dtype, device=band.device)
    e = torch.empty(max(n - 1, 0), dtype=band.dtype, device=band.device)
    s = stream if stream is not None else torch.cuda.current_stream(band.device)
    bb_sym_reduce(band.data_ptr(), band.stride(0), n, bw, tw, dt, d.data_ptr(), e.data_ptr() if n > 1 else 0,
                  work.data_ptr(), work.numel(), tun, s.cuda_stream)
    if check:
        st = bb_sym_device_status(work.data_ptr(), n, bw, tw, dt, s.cuda_stream)
        if st != BB_OK:
            raise BBError(st, "bb_sym_reduce")
    return d, e
