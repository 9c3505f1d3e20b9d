"""ctypes binding of libbb.so: the C ABI of include/bb.h, same names.

Argument marshalling only; every step of the reduction runs in the HIP
kernels.  Loading fails loudly when the library has not been built: there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbb.so")

BB_F32, BB_F64, BB_F16 = 0, 1, 2
BB_OK, BB_ERR_ARG, BB_ERR_WORKSPACE, BB_ERR_HIP, BB_ERR_UNSUPPORTED, BB_ERR_TIMEOUT = range(6)
BB_SCHED_DEFAULT, BB_SCHED_STEP, BB_SCHED_PERSISTENT, BB_SCHED_GROUP, BB_SCHED_BARRIER = 0, 1, 2, 3, 4

# Every symbol include/bb.h declares.
EXPORTS = ("bb_plan", "bb_workspace_bytes", "bb_reduce", "bb_pack", "bb_run_pass", "bb_run_passes", "bb_extract",
           "bb_launch_plan", "bb_export_band",
           "bb_device_status", "bb_sym_workspace_bytes", "bb_sym_reduce", "bb_sym_export_band",
           "bb_sym_device_status", "bb_svals_workspace_bytes", "bb_svals", "bb_svals_split", "bb_status_str",
           "bb_probe_stream", "bb_probe_transpose_add", "bb_probe_norm_clocks", "bb_reduce_noalloc")


class bb_tuning(ctypes.Structure):
    _fields_ = [("scheduler", ctypes.c_int32), ("stagger", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("threads_per_block", ctypes.c_int32), ("spin_limit", ctypes.c_int64),
                ("group_sweeps", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class bb_plan_info(ctypes.Structure):
    _fields_ = [("passes", ctypes.c_int32), ("ld", ctypes.c_int32), ("sub", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("sweeps", ctypes.c_int64), ("cycles", ctypes.c_int64),
                ("steps", ctypes.c_int64), ("alg_bytes", ctypes.c_double), ("flops", ctypes.c_double)]


class BBError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


_lib = None


def hip_runtimes(maps_text: str) -> list[str]:
    """Distinct HIP runtime files (libamdhip64) mapped, from /proc/self/maps text."""
    out = set()
    for line in maps_text.splitlines():
        parts = line.split()
        if len(parts) >= 6 and "libamdhip64" in os.path.basename(parts[-1]) and parts[-1].startswith("/"):
            out.add(os.path.realpath(parts[-1]))
    return sorted(out)


def check_one_runtime() -> None:
    """Raises when more than one HIP runtime is mapped into this process:
    launches would then go to a runtime that sees no device."""
    try:
        with open("/proc/self/maps") as fh:
            rts = hip_runtimes(fh.read())
    except OSError:
        return
    if len(rts) > 1:
        raise RuntimeError("more than one HIP runtime is loaded in this process (" + ", ".join(rts) + "); "
                           "import torch before loading any other HIP library, so that libbb.so binds to "
                           "torch's runtime")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built; run __graft_entry__.build()")
        # torch's HIP runtime must be loaded before this library's: loaded the
        # other way round, torch binds to the system runtime and the library's
        # first launch fails with hipErrorNoDevice
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        check_one_runtime()
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        L.bb_plan.argtypes = [i64, i32, i32, i32, ctypes.POINTER(bb_plan_info)]
        L.bb_workspace_bytes.argtypes = [i64, i32, i32, i32, ctypes.POINTER(sz)]
        L.bb_reduce.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, sz, ctypes.POINTER(bb_tuning), vp]
        L.bb_pack.argtypes = [vp, i64, i64, i32, i32, i32, vp, sz, vp]
        L.bb_run_pass.argtypes = [i64, i32, i32, i32, i32, vp, sz, ctypes.POINTER(bb_tuning), vp]
        L.bb_run_passes.argtypes = [i64, i32, i32, i32, i32, i32, vp, sz, ctypes.POINTER(bb_tuning), vp]
        L.bb_launch_plan.argtypes = [i64, i32, i32, i32, ctypes.POINTER(bb_tuning), ctypes.POINTER(i32), i32,
                                     ctypes.POINTER(i32)]
        L.bb_extract.argtypes = [vp, sz, i64, i32, i32, i32, vp, vp, vp]
        L.bb_export_band.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        L.bb_device_status.argtypes = [vp, i64, i32, i32, i32, vp]
        L.bb_sym_workspace_bytes.argtypes = [i64, i32, i32, i32, ctypes.POINTER(sz)]
        L.bb_sym_reduce.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, sz, ctypes.POINTER(bb_tuning), vp]
        L.bb_sym_export_band.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        L.bb_sym_device_status.argtypes = [vp, i64, i32, i32, i32, vp]
        L.bb_svals_workspace_bytes.argtypes = [i64, i32, ctypes.POINTER(sz)]
        L.bb_svals.argtypes = [vp, vp, i64, i32, i64, i64, i32, i32, vp, vp, sz, vp]
        L.bb_svals_split.argtypes = [i64, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.bb_reduce_noalloc.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, ctypes.POINTER(bb_tuning), vp]
        L.bb_probe_stream.argtypes = [vp, vp, vp, i64, i32, vp]
        L.bb_probe_transpose_add.argtypes = [vp, vp, i32, i32, vp]
        L.bb_probe_norm_clocks.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.bb_status_str.argtypes = [i32]
        L.bb_status_str.restype = ctypes.c_char_p
        for f in ("bb_plan", "bb_workspace_bytes", "bb_reduce", "bb_pack", "bb_run_pass", "bb_run_passes",
                  "bb_launch_plan", "bb_extract",
                  "bb_export_band", "bb_device_status", "bb_sym_workspace_bytes", "bb_sym_reduce",
                  "bb_sym_export_band", "bb_sym_device_status", "bb_svals_workspace_bytes", "bb_svals", "bb_svals_split",
                  "bb_probe_stream", "bb_probe_transpose_add", "bb_probe_norm_clocks", "bb_reduce_noalloc"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().bb_status_str(status).decode()


def bb_plan(n: int, bw: int, tw: int, dtype: int) -> bb_plan_info:
    out = bb_plan_info()
    rc = lib().bb_plan(n, bw, tw, dtype, ctypes.byref(out))
    if rc != BB_OK:
        raise BBError(rc, "bb_plan")
    return out


def bb_workspace_bytes(n: int, bw: int, tw: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().bb_workspace_bytes(n, bw, tw, dtype, ctypes.byref(out))
    if rc != BB_OK:
        raise BBError(rc, "bb_workspace_bytes")
    return int(out.value)


def bb_reduce(band_ptr: int, ld_band: int, n: int, bw: int, tw: int, dtype: int, d_ptr: int, e_ptr: int,
              work_ptr: int, work_bytes: int, tuning: bb_tuning | None, stream: int) -> None:
    rc = lib().bb_reduce(band_ptr, ld_band, n, bw, tw, dtype, d_ptr, e_ptr or None, work_ptr, work_bytes,
                         ctypes.byref(tuning) if tuning is not None else None, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_reduce")


BB_NOALLOC_SCRATCH_BYTES = 16 << 20


def bb_reduce_noalloc(band_ptr: int, ld_band: int, n: int, bw: int, tw: int, dtype: int, d_ptr: int, e_ptr: int,
                      status_ptr: int, tuning: bb_tuning | None, stream: int) -> None:
    rc = lib().bb_reduce_noalloc(band_ptr, ld_band, n, bw, tw, dtype, d_ptr, e_ptr or None, status_ptr or None,
                                 ctypes.byref(tuning) if tuning is not None else None, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_reduce_noalloc")


def bb_pack(band_ptr: int, ld_band: int, n: int, bw: int, tw: int, dtype: int, work_ptr: int, work_bytes: int,
            stream: int) -> None:
    rc = lib().bb_pack(band_ptr, ld_band, n, bw, tw, dtype, work_ptr, work_bytes, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_pack")


def bb_run_pass(n: int, bw: int, tw: int, dtype: int, pass_index: int, work_ptr: int, work_bytes: int,
                tuning: bb_tuning | None, stream: int) -> None:
    rc = lib().bb_run_pass(n, bw, tw, dtype, pass_index, work_ptr, work_bytes,
                           ctypes.byref(tuning) if tuning is not None else None, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_run_pass")


def bb_run_passes(n: int, bw: int, tw: int, dtype: int, first: int, count: int, work_ptr: int, work_bytes: int,
                  tuning: bb_tuning | None, stream: int) -> None:
    rc = lib().bb_run_passes(n, bw, tw, dtype, first, count, work_ptr, work_bytes,
                             ctypes.byref(tuning) if tuning is not None else None, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_run_passes")


def bb_launch_plan(n: int, bw: int, tw: int, dtype: int, tuning: bb_tuning | None) -> list[int]:
    """Index of the cycle-kernel launch that runs each pass (-1: no sweeps)."""
    passes = bb_plan(n, bw, tw, dtype).passes
    out = (ctypes.c_int32 * max(passes, 1))()
    count = ctypes.c_int32(0)
    rc = lib().bb_launch_plan(n, bw, tw, dtype, ctypes.byref(tuning) if tuning is not None else None, out,
                              passes, ctypes.byref(count))
    if rc != BB_OK:
        raise BBError(rc, "bb_launch_plan")
    return [int(out[i]) for i in range(passes)]


def bb_extract(work_ptr: int, work_bytes: int, n: int, bw: int, tw: int, dtype: int, d_ptr: int, e_ptr: int,
               stream: int) -> None:
    rc = lib().bb_extract(work_ptr, work_bytes, n, bw, tw, dtype, d_ptr, e_ptr or None, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_extract")


def bb_export_band(work_ptr: int, n: int, bw: int, tw: int, dtype: int, dst_ptr: int, stream: int) -> None:
    rc = lib().bb_export_band(work_ptr, n, bw, tw, dtype, dst_ptr, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_export_band")


def bb_device_status(work_ptr: int, n: int, bw: int, tw: int, dtype: int, stream: int) -> int:
    return int(lib().bb_device_status(work_ptr, n, bw, tw, dtype, stream or None))


def bb_sym_workspace_bytes(n: int, bw: int, tw: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().bb_sym_workspace_bytes(n, bw, tw, dtype, ctypes.byref(out))
    if rc != BB_OK:
        raise BBError(rc, "bb_sym_workspace_bytes")
    return int(out.value)


def bb_sym_reduce(band_ptr: int, ld_band: int, n: int, bw: int, tw: int, dtype: int, d_ptr: int, e_ptr: int,
                  work_ptr: int, work_bytes: int, tuning: bb_tuning | None, stream: int) -> None:
    rc = lib().bb_sym_reduce(band_ptr, ld_band, n, bw, tw, dtype, d_ptr, e_ptr or None, work_ptr, work_bytes,
                             ctypes.byref(tuning) if tuning is not None else None, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_sym_reduce")


def bb_sym_export_band(work_ptr: int, n: int, bw: int, tw: int, dtype: int, dst_ptr: int, stream: int) -> None:
    rc = lib().bb_sym_export_band(work_ptr, n, bw, tw, dtype, dst_ptr, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_sym_export_band")


def bb_sym_device_status(work_ptr: int, n: int, bw: int, tw: int, dtype: int, stream: int) -> int:
    return int(lib().bb_sym_device_status(work_ptr, n, bw, tw, dtype, stream or None))


def bb_svals_workspace_bytes(n: int, dtype: int) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().bb_svals_workspace_bytes(n, dtype, ctypes.byref(out))
    if rc != BB_OK:
        raise BBError(rc, "bb_svals_workspace_bytes")
    return int(out.value)


def bb_svals(d_ptr: int, e_ptr: int, n: int, dtype: int, i0: int, i1: int, tree_levels: int, levels: int,
             sigma_ptr: int, work_ptr: int, work_bytes: int, stream: int) -> None:
    rc = lib().bb_svals(d_ptr or None, e_ptr or None, n, dtype, i0, i1, tree_levels, levels, sigma_ptr or None,
                        work_ptr or None, work_bytes, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_svals")


def bb_svals_split(values: int, dtype: int):
    """(tree_levels, levels) that bb_svals picks for this many values."""
    k, d = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = lib().bb_svals_split(values, dtype, ctypes.byref(k), ctypes.byref(d))
    if rc != BB_OK:
        raise BBError(rc, "bb_svals_split")
    return int(k.value), int(d.value)


def bb_probe_stream(x_ptr: int, y_ptr: int, z_ptr: int, n: int, reps: int, stream: int) -> None:
    rc = lib().bb_probe_stream(x_ptr, y_ptr, z_ptr, n, reps, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_probe_stream")


def bb_probe_transpose_add(a_ptr: int, b_ptr: int, m: int, reps: int, stream: int) -> None:
    rc = lib().bb_probe_transpose_add(a_ptr, b_ptr, m, reps, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_probe_transpose_add")


def bb_probe_norm_clocks(m: int, mode: int, reps: int, x_ptr: int, out_ptr: int, clocks_ptr: int,
                         stream: int) -> None:
    rc = lib().bb_probe_norm_clocks(m, mode, reps, x_ptr, out_ptr, clocks_ptr, stream or None)
    if rc != BB_OK:
        raise BBError(rc, "bb_probe_norm_clocks")


def bb_status_str(status: int) -> str:
    return status_str(status)
