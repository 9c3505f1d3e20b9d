"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

* libbb.so loads and exports every function include/bb.h declares;
* bb_plan agrees with an independent enumeration of passes, sweeps and
  cycles, and with the closed form of the algorithmic bytes per cycle;
* invalid arguments are rejected on the host before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

import band_bidiagonal_bulge_amd as bbm
from band_bidiagonal_bulge_amd import _lib
from refs import cycles_of_sweep, pass_list

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "bb.h")).read()
    return sorted(set(re.findall(r"^\s*(?:bb_status|const char \*)\s*(bb_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for name in names:
        assert hasattr(L, name), name
    nm = os.popen("nm -D --defined-only " + _lib.LIB_PATH).read()
    for name in names:
        assert re.search(r"\bT " + name + r"\b", nm), name


def test_status_strings():
    for s in range(6):
        assert bbm.bb_status_str(s) and bbm.bb_status_str(s) != "unknown status"
    assert bbm.bb_status_str(99) == "unknown status"


def _enumerate(n, bw, tw, esize):
    cycles = sweeps = 0
    nbytes = 0.0
    for (b, t) in pass_list(bw, tw):
        bp = b - t
        ns = max(n - bp - 1, 0)
        sweeps += ns
        for R in range(ns):
            K = cycles_of_sweep(n, b, t, R)
            cycles += K
            for k in range(K):
                c = R + bp + k * b
                ch = min(c + t, n - 1)
                r = R if k == 0 else c - b
                m = ch - c + 1
                rows = ch - r + 1
                cols = min(c + t + b, n - 1) - c + 1
                nbytes += 2 * m * (rows + cols - m) * esize
    return sweeps, cycles, nbytes


@pytest.mark.parametrize("n,bw,tw,dt", [(512, 16, 8, 1), (300, 33, 7, 0), (97, 10, 20, 1), (5, 4, 2, 0)])
def test_plan_matches_enumeration(n, bw, tw, dt):
    info = bbm.bb_plan(n, bw, tw, dt)
    sweeps, cycles, nbytes = _enumerate(n, bw, tw, 8 if dt == 1 else 4)
    assert info.passes == len(pass_list(bw, tw))
    assert info.sweeps == sweeps and info.cycles == cycles
    assert abs(info.alg_bytes - nbytes) <= 1e-9 * nbytes
    t0 = min(tw, bw - 1) if bw > 1 else 0
    assert info.sub == t0 and info.ld == 2 * t0 + bw + 1


def test_plan_headline_workload_counts():
    # n = 16384, BW 64 -> 48 -> 32 -> 16 -> 1 with TW = 16, fp32
    info = bbm.bb_plan(16384, 64, 16, 0)
    assert info.passes == 4
    assert info.sweeps == 16335 + 16351 + 16367 + 16382
    assert info.cycles == 2092800 + 2793131 + 4193792 + 8394752
    assert abs(info.alg_bytes / 1e9 - (41.11 + 42.78 + 46.07 + 51.47)) < 0.02


def test_workspace_bytes_cover_band_and_counters():
    n, bw, tw = 1000, 20, 6
    nb = bbm.bb_workspace_bytes(n, bw, tw, 1)
    info = bbm.bb_plan(n, bw, tw, 1)
    assert nb >= n * info.ld * 8 + 128 * n
    assert nb % 256 == 0


def test_invalid_arguments_rejected_on_host():
    L = _lib.lib()
    sz = ctypes.c_size_t(0)
    assert L.bb_workspace_bytes(0, 4, 2, 0, ctypes.byref(sz)) == _lib.BB_ERR_ARG
    assert L.bb_workspace_bytes(10, -1, 2, 0, ctypes.byref(sz)) == _lib.BB_ERR_ARG
    assert L.bb_workspace_bytes(10, 4, 0, 0, ctypes.byref(sz)) == _lib.BB_ERR_ARG
    assert L.bb_workspace_bytes(10, 4, 2, 7, ctypes.byref(sz)) == _lib.BB_ERR_ARG
    assert L.bb_workspace_bytes(10, 4, 2, 0, None) == _lib.BB_ERR_ARG
    assert L.bb_workspace_bytes(1000, 200, 100, 0, ctypes.byref(sz)) == _lib.BB_ERR_UNSUPPORTED
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    # null band / d / e / work
    assert L.bb_reduce(None, 5, 10, 4, 2, 0, fake, fake, fake, 1 << 20, None, None) == _lib.BB_ERR_ARG
    assert L.bb_reduce(fake, 5, 10, 4, 2, 0, None, fake, fake, 1 << 20, None, None) == _lib.BB_ERR_ARG
    assert L.bb_reduce(fake, 5, 10, 4, 2, 0, fake, None, fake, 1 << 20, None, None) == _lib.BB_ERR_ARG
    assert L.bb_reduce(fake, 5, 10, 4, 2, 0, fake, fake, None, 1 << 20, None, None) == _lib.BB_ERR_ARG
    # ld_band too small, misaligned pointers, workspace too small
    assert L.bb_reduce(fake, 4, 10, 4, 2, 0, fake, fake, fake, 1 << 20, None, None) == _lib.BB_ERR_ARG
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L.bb_reduce(odd, 5, 10, 4, 2, 0, fake, fake, fake, 1 << 20, None, None) == _lib.BB_ERR_ARG
    assert L.bb_reduce(fake, 5, 10, 4, 2, 0, fake, fake, fake, 16, None, None) == _lib.BB_ERR_WORKSPACE
    # bad tuning
    for bad in (_lib.bb_tuning(9, 0, 0, 0, 0), _lib.bb_tuning(1, 1, 0, 0, 0), _lib.bb_tuning(1, 0, 0, 100, 0),
                _lib.bb_tuning(1, 0, -1, 0, 0), _lib.bb_tuning(1, 0, 0, 0, -5)):
        assert L.bb_reduce(fake, 5, 10, 4, 2, 0, fake, fake, fake, 1 << 20, ctypes.byref(bad), None) == \
            _lib.BB_ERR_ARG
    # n = 1 needs no e
    assert L.bb_reduce(fake, 5, 1, 4, 2, 0, fake, None, fake, 16, None, None) == _lib.BB_ERR_WORKSPACE


def test_staged_entry_points_validate_on_host():
    L = _lib.lib()
    fake = ctypes.c_void_p(1 << 20)
    big = 1 << 30
    # bb_pack: null band, short ld_band, small workspace, misaligned work
    assert L.bb_pack(None, 5, 10, 4, 2, 0, fake, big, None) == _lib.BB_ERR_ARG
    assert L.bb_pack(fake, 4, 10, 4, 2, 0, fake, big, None) == _lib.BB_ERR_ARG
    assert L.bb_pack(fake, 5, 10, 4, 2, 0, fake, 16, None) == _lib.BB_ERR_WORKSPACE
    assert L.bb_pack(fake, 5, 10, 4, 2, 0, ctypes.c_void_p((1 << 20) + 8), big, None) == _lib.BB_ERR_ARG
    # bb_run_pass: pass index out of range (10, 4, 2 has passes 4->2->1)
    assert bbm.bb_plan(10, 4, 2, 0).passes == 2
    for bad_pass in (-1, 2, 100):
        assert L.bb_run_pass(10, 4, 2, 0, bad_pass, fake, big, None, None) == _lib.BB_ERR_ARG
    assert L.bb_run_pass(10, 4, 2, 0, 0, fake, 16, None, None) == _lib.BB_ERR_WORKSPACE
    bad = _lib.bb_tuning(9, 0, 0, 0, 0)
    assert L.bb_run_pass(10, 4, 2, 0, 0, fake, big, ctypes.byref(bad), None) == _lib.BB_ERR_ARG
    # bb_run_passes: the range must lie within the passes; an empty range
    # launches nothing
    for (first, count) in ((-1, 1), (0, -1), (0, 3), (2, 1), (1, 2)):
        assert L.bb_run_passes(10, 4, 2, 0, first, count, fake, big, None, None) == _lib.BB_ERR_ARG
    assert L.bb_run_passes(10, 4, 2, 0, 1, 0, fake, big, None, None) == _lib.BB_OK
    assert L.bb_run_passes(10, 4, 2, 0, 0, 2, fake, 16, None, None) == _lib.BB_ERR_WORKSPACE
    # bb_extract: null d, null e with n > 1, misaligned d
    assert L.bb_extract(fake, big, 10, 4, 2, 0, None, fake, None) == _lib.BB_ERR_ARG
    assert L.bb_extract(fake, big, 10, 4, 2, 0, fake, None, None) == _lib.BB_ERR_ARG
    assert L.bb_extract(fake, big, 10, 4, 2, 1, ctypes.c_void_p((1 << 20) + 4), fake, None) == _lib.BB_ERR_ARG


def test_svals_validation_without_a_gpu():
    # argument errors are reported before anything touches a device
    import ctypes
    L = bbm.lib()
    fake = ctypes.c_void_p(1 << 20)
    big = 1 << 24
    cases = [
        ((fake, fake, -1, 0, 0, 0, 0, 0, fake, fake, big, None), 1),
        ((fake, fake, 8, 2, 0, 1, 0, 0, fake, fake, big, None), 1),     # bad dtype
        ((fake, fake, 8, 0, 0, 9, 0, 0, fake, fake, big, None), 1),     # i1 > n
        ((fake, fake, 8, 0, 3, 2, 0, 0, fake, fake, big, None), 1),     # i1 < i0
        ((fake, fake, 8, 0, 0, 8, 0, 7, fake, fake, big, None), 1),     # levels
        ((fake, fake, 8, 0, 0, 8, 17, 0, fake, fake, big, None), 1),    # tree levels
        ((fake, fake, 8, 0, 0, 8, -2, 0, fake, fake, big, None), 1),    # tree levels
        ((None, fake, 8, 0, 0, 8, 0, 0, fake, fake, big, None), 1),     # d NULL
        ((fake, fake, 8, 0, 0, 8, 0, 0, fake, fake, 16, None), 2),      # workspace
        ((fake, fake, 1 << 30, 0, 0, 1, 0, 0, fake, fake, 1 << 40, None), 1),  # n too large
        ((None, None, 0, 0, 0, 0, 0, 0, None, None, 0, None), 0),       # nothing to do
        ((None, None, 8, 0, 4, 4, 0, 0, None, None, 0, None), 0),       # empty range
    ]
    for args, want in cases:
        assert L.bb_svals(*args) == want, args
    assert bbm.bb_svals_workspace_bytes(16384, 0) == 256 + (4 << 16) + (32768 + 64) * 4
    assert bbm.bb_svals_workspace_bytes(1, 1) == 256 + (4 << 16) + 128 * 8
    with pytest.raises(bbm.BBError):
        bbm.bb_svals_workspace_bytes(-1, 0)
    # split for the size (256 CUs when no device answers): the 16 shared tree
    # levels fill 1024 SIMDs in one round; then 2 levels per round with 4 lanes
    # per value fill them again at 16384 values
    assert bbm.bb_svals_split(16384, 0) == (16, 2)
    # one value: the deepest rounds, and the smallest tree that reaches the
    # same round count (55 halvings = 13 tree levels + 7 rounds of 6)
    assert bbm.bb_svals_split(1, 1) == (13, 6)


def test_sym_and_f16_validation_without_a_gpu():
    import ctypes
    L = bbm.lib()
    fake = ctypes.c_void_p(1 << 20)
    sz = ctypes.c_size_t(0)
    # the symmetric reduction takes fp32 and fp64 only
    assert L.bb_sym_workspace_bytes(100, 8, 4, 2, ctypes.byref(sz)) == 4
    assert L.bb_sym_workspace_bytes(100, 8, 4, 0, ctypes.byref(sz)) == 0 and sz.value > 0
    assert L.bb_sym_reduce(fake, 9, 100, 8, 4, 2, fake, fake, fake, 1 << 30, None, None) == 4
    assert L.bb_sym_export_band(fake, 100, 8, 4, 2, fake, None) == 4
    # half precision is a valid dtype of the general reduction
    info = bbm.bb_plan(100, 8, 4, bbm.BB_F16)
    assert info.passes == 2
    assert bbm.bb_workspace_bytes(100, 8, 4, bbm.BB_F16) < bbm.bb_workspace_bytes(100, 8, 4, bbm.BB_F32)
    # STEP has no fp16 kernel: rejected before anything is enqueued
    tun = bbm.tuning(scheduler=bbm.BB_SCHED_STEP)
    ws = bbm.bb_workspace_bytes(100, 8, 4, bbm.BB_F16)
    assert L.bb_run_pass(100, 8, 4, 2, 0, ctypes.c_void_p(1 << 20), ws, ctypes.byref(tun), None) == 4


def test_launch_plan_groups_consecutive_passes():
    # which cycle-kernel launch runs each pass (host only): under the default
    # scheduler consecutive group-kernel passes with one tile family share a
    # launch, at most four; the other schedulers launch once per pass; passes
    # without sweeps launch nothing
    plan = bbm.bb_launch_plan
    sched = [bbm.tuning(scheduler=s) for s in (bbm.BB_SCHED_DEFAULT, bbm.BB_SCHED_STEP, bbm.BB_SCHED_PERSISTENT,
                                               bbm.BB_SCHED_GROUP)]
    assert plan(16384, 64, 16, bbm.BB_F32, sched[0]) == [0, 0, 0, 0]        # tiles 17, 17, 17, 16
    assert plan(16384, 64, 16, bbm.BB_F16, sched[0]) == [0, 0, 0, 0]
    assert plan(512, 16, 8, bbm.BB_F64, sched[0]) == [0, 0]                  # tiles 9, 8
    for tun in sched[1:]:
        assert plan(16384, 64, 16, bbm.BB_F32, tun) == [0, 1, 2, 3]
    assert plan(600, 64, 4, bbm.BB_F32, sched[0]) == sum(([k] * 4 for k in range(4)), [])  # 16 passes
    assert plan(4096, 64, 15, bbm.BB_F32, sched[0]) == [0, 0, 0, 0, 1]     # tiles 16 x 4, then 9 (t = 3)
    assert plan(32768, 128, 32, bbm.BB_F64, sched[0]) == [0, 1, 2, 3]      # t + 1 = 33: persistent
    assert plan(5, 8, 2, bbm.BB_F32, sched[0]) == [-1, -1, 0, 0]           # b' >= n - 1: no sweeps
    L = _lib.lib()
    count = ctypes.c_int32(-1)
    assert L.bb_launch_plan(16384, 64, 16, 0, None, None, 0, ctypes.byref(count)) == _lib.BB_OK
    assert count.value == 1
    out = (ctypes.c_int32 * 4)()
    assert L.bb_launch_plan(16384, 64, 16, 0, None, out, 3, ctypes.byref(count)) == _lib.BB_ERR_ARG
    assert L.bb_launch_plan(16384, 64, 16, 0, None, out, 4, None) == _lib.BB_ERR_ARG
    assert L.bb_launch_plan(16384, 64, 16, 2, ctypes.byref(sched[1]), out, 4, ctypes.byref(count)) == \
        _lib.BB_ERR_UNSUPPORTED


def test_hip_runtime_parser_finds_duplicates():
    # /proc/self/maps text: one runtime mapped twice (several segments) is
    # one; two different files are two
    from band_bidiagonal_bulge_amd._lib import hip_runtimes
    one = ("7f00-7f10 r-xp 00000000 00:2a 11 /opt/t/lib/libamdhip64.so\n"
           "7f10-7f20 r--p 00010000 00:2a 11 /opt/t/lib/libamdhip64.so\n"
           "7f20-7f30 r-xp 00000000 00:2a 12 /usr/lib/libc.so.6\n")
    assert hip_runtimes(one) == ["/opt/t/lib/libamdhip64.so"]
    two = one + "7f40-7f50 r-xp 00000000 00:2a 13 /opt/rocm/lib/libamdhip64.so.7\n"
    assert len(hip_runtimes(two)) == 2
    assert hip_runtimes("7f00-7f10 rw-p 00000000 00:00 0 \n") == []


def test_wait_bound_is_validated():
    # the per-wait bound is in microseconds, at most twenty seconds
    import band_bidiagonal_bulge_amd as bbm
    assert bbm.bb_launch_plan(1000, 32, 16, bbm.BB_F32, bbm.tuning(spin_limit=20000000))
    with pytest.raises(bbm.BBError):
        bbm.bb_launch_plan(1000, 32, 16, bbm.BB_F32, bbm.tuning(spin_limit=20000001))
    with pytest.raises(bbm.BBError):
        bbm.bb_launch_plan(1000, 32, 16, bbm.BB_F32, bbm.tuning(spin_limit=-1))
