"""Parity of the HIP path with the CPU oracle, through the C ABI (needs a GPU).

The kernels follow the same arithmetic contract as the oracle (serial sums in
increasing index, explicit fused multiply-adds, correctly rounded sqrt and
division), so on every case here the GPU result is compared to the bit with
the oracle's, on top of the tolerance gates: |d|, |e| elementwise within
1e-10 ||A||_F (fp64) or 2e-4 ||A||_F (fp32), singular values within the same
bound, exact zeros off the bidiagonal.
"""
import hashlib
import os

import numpy as np
import pytest

import band_bidiagonal_bulge_amd as bbm
import bb_inputs
import oracle
from gpu_util import TOL, assert_bits_equal, gpu_reduce, log, weyl_sv_bound
from refs import bidiag_singular_values

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# (n, bw, tw, dtype, dist): several tiles, ragged tails, every register tile
# size (t+1 = 9, 17, 33, 65), single-cycle sweeps, TW >= BW, one pass, and
# passes with b' = 1, 2 and >= 3 (each a different wait between sweeps).
SMALL = [
    (512, 16, 8, "f64", "normal"),
    (1000, 32, 16, "f32", "normal"),
    (777, 24, 5, "f64", "normal"),
    (300, 64, 16, "f32", "normal"),
    (257, 33, 32, "f32", "uniform"),
    (200, 65, 64, "f64", "normal"),
    (301, 128, 32, "f32", "normal"),
    (130, 10, 3, "f32", "normal"),
    (97, 9, 40, "f64", "normal"),
    (40, 39, 13, "f64", "normal"),
    (17, 16, 5, "f32", "normal"),
    (500, 256, 32, "f32", "uniform_zero_rows"),
    (500, 18, 16, "f32", "normal"),   # a b' = 2 pass (18 -> 2), then 2 -> 1
    (400, 12, 10, "f64", "normal"),   # the same in fp64 (12 -> 2 -> 1)
    (300, 65, 16, "f32", "normal"),   # split halves with 64 early lanes (65 -> 49), then 49 -> 33
    (600, 64, 16, "f64", "normal"),   # split halves in fp64
]


def _check_bitwise(band, bw, tw, tun=None):
    n = band.shape[0]
    d, e, W, sub = gpu_reduce(band, bw, tw, tun, return_band=True)
    od, oe, OW, osub = oracle.reduce(band, bw, tw, return_band=True)
    assert sub == osub and W.shape == OW.shape
    assert_bits_equal(d, od)
    assert_bits_equal(e, oe)
    assert_bits_equal(W, OW)
    return d, e, W, sub


@pytest.mark.parametrize("n,bw,tw,dt,dist", SMALL)
def test_bitwise_equal_to_oracle(n, bw, tw, dt, dist):
    log(f"bitwise n={n} bw={bw} tw={tw} {dt} {dist}")
    band = bb_inputs.make_band(n, bw, dt, dist, seed=n + bw)
    d, e, W, sub = _check_bitwise(band, bw, tw)
    off = [o for o in range(W.shape[1]) if o - sub not in (0, 1)]
    assert np.all(W[:, off] == 0)


@pytest.mark.parametrize("n,bw,tw", [(1, 3, 1), (2, 4, 2), (3, 2, 1), (50, 0, 4), (50, 1, 4), (64, 2, 1)])
@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_degenerate_shapes(n, bw, tw, dt):
    log(f"degenerate n={n} bw={bw} tw={tw} {dt}")
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=7)
    _check_bitwise(band, bw, tw)


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_all_zero_and_zero_rows(dt):
    n, bw, tw = 400, 32, 16
    log(f"zero band {dt}")
    z = np.zeros((n, bw + 1), dtype=bb_inputs.np_dtype(dt))
    d, e, W, _ = _check_bitwise(z, bw, tw)
    assert np.all(W == 0)
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=3)
    band[[0, 1, 7, 15, 16, 200, 399], :] = 0
    log(f"zero rows {dt}")
    _check_bitwise(band, bw, tw)


STEP, PERSIST, GROUP, BARRIER = 1, 2, 3, 4


@pytest.mark.parametrize("tun", [dict(scheduler=STEP), dict(scheduler=STEP, stagger=3),
                                 dict(scheduler=STEP, threads_per_block=64),
                                 dict(scheduler=PERSIST), dict(scheduler=PERSIST, max_blocks=1),
                                 dict(scheduler=PERSIST, max_blocks=2), dict(scheduler=PERSIST, max_blocks=7),
                                 dict(scheduler=PERSIST, threads_per_block=64),
                                 dict(scheduler=PERSIST, threads_per_block=256, max_blocks=1000),
                                 dict(scheduler=GROUP), dict(scheduler=GROUP, group_sweeps=1),
                                 dict(scheduler=GROUP, group_sweeps=2, max_blocks=1),
                                 dict(scheduler=GROUP, group_sweeps=3, max_blocks=2),
                                 dict(scheduler=GROUP, group_sweeps=6, max_blocks=5),
                                 dict(scheduler=BARRIER), dict(scheduler=BARRIER, stagger=3),
                                 dict(scheduler=BARRIER, max_blocks=1),
                                 dict(scheduler=BARRIER, max_blocks=3, threads_per_block=64)])
@pytest.mark.parametrize("n,bw,tw,dt", [(900, 48, 16, "f32"), (700, 24, 7, "f64"), (400, 9, 2, "f32")])
def test_scheduler_variants_bitwise(tun, n, bw, tw, dt):
    log(f"variant {tun} n={n} bw={bw} tw={tw} {dt}")
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=5)
    _check_bitwise(band, bw, tw, bbm.tuning(**tun))


# Runs of passes in one launch (the default scheduler): every pass's first
# group starts on rows the previous pass has released while that pass still
# runs.  Shapes: four passes in one launch, runs split at four passes (BW 64 /
# TW 4: 16 passes), mixed tiles (t+1 = 9 then 8, 17 then 16), two rows per
# lane then one, fp16, a first pass with the smaller tile and two rows per
# lane (TW 15 and 7), persistent passes before a run (BW 128 and 100: their
# rings do not fit) and runs split where their groups would exceed the
# progress lines; few resident workgroups, where a pass's first group waits
# longest for the previous pass.
@pytest.mark.parametrize("tun", [dict(), dict(max_blocks=1), dict(max_blocks=3), dict(group_sweeps=2, max_blocks=5)])
@pytest.mark.parametrize("n,bw,tw,dt", [(900, 64, 16, "f32"), (700, 24, 7, "f64"), (600, 64, 4, "f32"),
                                        (300, 64, 8, "f32"), (800, 64, 16, "f16"), (640, 40, 13, "f64"),
                                        (500, 64, 15, "f32"), (300, 64, 7, "f16"), (1500, 128, 16, "f32"),
                                        (900, 100, 16, "f64")])
def test_fused_passes_bitwise(tun, n, bw, tw, dt):
    log(f"fused {tun} n={n} bw={bw} tw={tw} {dt}")
    launches = bbm.bb_launch_plan(n, bw, tw, {"f32": 0, "f64": 1, "f16": 2}[dt], bbm.tuning(**tun))
    assert len(set(launches)) < len(launches)  # some passes do share a launch
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=n + bw)
    _check_bitwise(band, bw, tw, bbm.tuning(**tun))


# The persistent kernel publishes each half's pivot and first t+1 rows or
# columns before the rest (the whole half for fp64 passes with b' <= 2):
# wide and narrow tiles, staged and unstaged row halves, workgroups smaller
# than the early part (64 threads, t+1 = 65), passes with b' = 1 and 2 in
# both precisions, identity reflectors (zero rows), ragged last cycles.
@pytest.mark.parametrize("n,bw,tw,dt,dist,nt", [(301, 128, 64, "f32", "normal", 64),
                                                (257, 96, 64, "f64", "normal", 0),
                                                (333, 40, 31, "f32", "normal", 0),
                                                (333, 40, 31, "f64", "normal", 128),
                                                (211, 18, 16, "f64", "normal", 0),
                                                (211, 18, 16, "f32", "normal", 64),
                                                (517, 128, 32, "f32", "uniform_zero_rows", 0),
                                                (517, 64, 32, "f64", "uniform_zero_rows", 192),
                                                (450, 48, 16, "f32", "normal", 0)])
def test_persistent_early_publication_bitwise(n, bw, tw, dt, dist, nt):
    log(f"persistent early publication n={n} bw={bw} tw={tw} {dt} {dist} threads={nt}")
    band = bb_inputs.make_band(n, bw, dt, dist, seed=n + tw)
    _check_bitwise(band, bw, tw, bbm.tuning(scheduler=PERSIST, threads_per_block=nt))


# Passes with t = 31 and b + t <= 64 (fp32 and fp64), or t = 32 and
# b + t <= 128 (fp32), run the group kernel on windows of the working band's
# rows (the band's full rows would leave room for one sweep per group):
# alone, after persistent passes, before a narrow pass, ragged, several group
# sizes, a pass of b = 33 (b' = 2), two rows per lane, zero rows.
@pytest.mark.parametrize("n,bw,tw,dt,tun", [(700, 32, 31, "f32", dict()),
                                            (517, 64, 31, "f32", dict()),
                                            (1000, 256, 32, "f32", dict()),
                                            (150, 32, 31, "f32", dict()),
                                            (611, 32, 31, "f32", dict(scheduler=GROUP, group_sweeps=3)),
                                            (611, 32, 31, "f32", dict(scheduler=GROUP, group_sweeps=6, max_blocks=2)),
                                            (444, 33, 31, "f32", dict(scheduler=GROUP, group_sweeps=4)),
                                            (700, 32, 31, "f64", dict()),
                                            (900, 64, 32, "f32", dict()),
                                            (700, 128, 32, "f32", dict()),
                                            (555, 96, 32, "f32", dict(scheduler=GROUP, group_sweeps=3)),
                                            (333, 64, 32, "f32", "uniform_zero_rows"),
                                            (444, 33, 31, "f64", dict()),
                                            (321, 32, 31, "f64", "uniform_zero_rows"),
                                            (600, 128, 32, "f64", dict(scheduler=GROUP))])
def test_windowed_group_passes_bitwise(n, bw, tw, dt, tun):
    log(f"windowed group n={n} bw={bw} tw={tw} {dt} {tun}")
    dist = tun if isinstance(tun, str) else "normal"
    tun = {} if isinstance(tun, str) else tun
    band = bb_inputs.make_band(n, bw, dt, dist, seed=n + 3)
    _check_bitwise(band, bw, tw, bbm.tuning(**tun))


@pytest.mark.parametrize("n,bw,tw,dt", [(500, 64, 32, "f64"), (300, 40, 31, "f32")])
def test_barrier_scheduler_wide_tiles_bitwise(n, bw, tw, dt):
    log(f"barrier scheduler n={n} bw={bw} tw={tw} {dt}")
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=6)
    _check_bitwise(band, bw, tw, bbm.tuning(scheduler=BARRIER))


def test_barrier_scheduler_refuses_half_precision():
    import torch
    band = torch.zeros(64, 9, dtype=torch.float16, device="cuda:0")
    with pytest.raises(bbm.BBError):
        bbm.reduce(band, 8, 4, bbm.tuning(scheduler=BARRIER))


@pytest.mark.parametrize("sched", [PERSIST, GROUP, bbm.BB_SCHED_DEFAULT, BARRIER])
def test_forced_timeout_reports_status(sched):
    # A spin limit of one poll makes the first wait on a predecessor expire;
    # every workgroup then stops and the launch ends normally.
    import torch
    n, bw, tw = 3000, 32, 16
    band = torch.from_numpy(bb_inputs.make_band(n, bw, "f32", "normal", seed=2)).to("cuda:0")
    work = bbm.workspace(n, bw, tw, band.dtype)
    log(f"forced timeout sched={sched}")
    bbm.reduce(band, bw, tw, bbm.tuning(scheduler=sched, spin_limit=1), work)
    st = bbm.bb_device_status(work.data_ptr(), n, bw, tw, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 5, bbm.bb_status_str(st)
    # the next normal call on the same workspace clears the status
    d, e = bbm.reduce(band, bw, tw, None, work)
    st = bbm.bb_device_status(work.data_ptr(), n, bw, tw, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    od, oe = oracle.reduce(band.cpu().numpy(), bw, tw)
    assert_bits_equal(d.cpu().numpy(), od)


def test_forced_timeout_drains_the_launch():
    # Every wait bounded to 1 us on the headline band, all four passes in one
    # launch: the first wait that is not satisfied at once expires, every
    # other wait and every claim then sees the status word, and the launch
    # drains well inside a second; the next call succeeds.
    import time
    import torch
    n, bw, tw = 16384, 64, 16
    band = torch.from_numpy(bb_inputs.make_band(n, bw, "f32", "normal", seed=0)).to("cuda:0")
    work = bbm.workspace(n, bw, tw, band.dtype)
    bbm.reduce(band, bw, tw, None, work)
    torch.cuda.synchronize()
    log("forced timeout, headline band, one launch")
    t0 = time.perf_counter()
    bbm.reduce(band, bw, tw, bbm.tuning(spin_limit=1), work)
    st = bbm.bb_device_status(work.data_ptr(), n, bw, tw, 0, torch.cuda.current_stream().cuda_stream)
    dt = time.perf_counter() - t0
    assert st == bbm.BB_ERR_TIMEOUT, bbm.bb_status_str(st)
    assert dt < 1.0, dt
    with pytest.raises(bbm.BBError):
        bbm.reduce(band, bw, tw, bbm.tuning(spin_limit=1), work, check=True)
    d, e = bbm.reduce(band, bw, tw, None, work, check=True)
    z = np.load(os.path.join(GOLDEN, "n16384-bw64-tw16-f32-normal.npz"))
    assert_bits_equal(d.cpu().numpy(), z["d"], "d")


def test_library_loaded_before_torch():
    # a fresh process whose first call is host-only (it loads libbb.so before
    # torch has been imported) still reduces on the GPU: the binding imports
    # torch's HIP runtime first
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys\n"
        "import band_bidiagonal_bulge_amd as bbm\n"
        "assert 'torch' not in sys.modules\n"
        "plan = bbm.bb_launch_plan(300, 24, 8, bbm.BB_F32, None)\n"
        "import numpy as np, torch, bb_inputs\n"
        "band = bb_inputs.make_band(300, 24, 'f32', 'normal', seed=4)\n"
        "d, e = bbm.reduce(torch.from_numpy(band).to('cuda:0'), 24, 8)\n"
        "torch.cuda.synchronize()\n"
        "print('ok', plan, float(d.double().abs().sum()))\n")
    log("fresh process: library loaded before torch")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=240,
                       env=dict(os.environ, PYTHONPATH=root))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.startswith("ok")


def test_repeated_calls_reuse_workspace():
    n, bw, tw = 600, 40, 12
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=9)
    log("repeat x3")
    d, e = gpu_reduce(band, bw, tw, reps=3)
    od, oe = oracle.reduce(band, bw, tw)
    assert_bits_equal(d, od)
    assert_bits_equal(e, oe)


def _gate(w, d, e, od, oe, fro):
    tol = TOL[w.dtype] * fro
    assert np.all(np.isfinite(d)) and np.all(np.isfinite(e))
    assert np.max(np.abs(np.abs(d) - np.abs(od))) <= tol
    assert np.max(np.abs(np.abs(e) - np.abs(oe))) <= tol
    assert weyl_sv_bound(d, e, od, oe) <= tol
    f2 = np.sum(d.astype(np.float64) ** 2) + np.sum(e.astype(np.float64) ** 2)
    assert abs(f2 - fro * fro) <= (1e-12 if w.dtype == "f64" else 1e-5) * fro * fro


@pytest.mark.parametrize("name", ["n512-bw16-tw8-f64-normal", "n4096-bw32-tw16-f32-normal"])
def test_workload_live_oracle(name):
    w = bb_inputs.WORKLOADS[name]
    band = bb_inputs.make_workload(w)
    fro = float(np.linalg.norm(band.astype(np.float64)))
    log(f"workload {name}")
    d, e, W, sub = gpu_reduce(band, w.bw, w.tw, return_band=True)
    od, oe = oracle.reduce(band, w.bw, w.tw)
    _gate(w, d, e, od, oe, fro)
    assert_bits_equal(d, od)
    assert_bits_equal(e, oe)
    off = [o for o in range(W.shape[1]) if o - sub not in (0, 1)]
    assert np.all(W[:, off] == 0)
    sv = bidiag_singular_values(d, e)
    osv = bidiag_singular_values(od, oe)
    assert np.max(np.abs(sv - osv)) <= TOL[w.dtype] * fro


@pytest.mark.parametrize("name", ["n16384-bw64-tw16-f32-normal", "n32768-bw128-tw32-f64-graded",
                                  "n65536-bw256-tw32-f32-zerorows"])
def test_workload_stored_oracle(name):
    path = os.path.join(GOLDEN, name + ".npz")
    if not os.path.exists(path):
        pytest.skip("stored oracle output not generated for " + name)
    z = np.load(path)
    w = bb_inputs.WORKLOADS[name]
    band = bb_inputs.make_workload(w)
    assert hashlib.sha256(band.tobytes()).hexdigest() == str(z["input_sha"]), "input generator drifted"
    fro = float(z["fro"])
    log(f"workload {name}")
    d, e, W, sub = gpu_reduce(band, w.bw, w.tw, return_band=True)
    _gate(w, d, e, z["d"], z["e"], fro)
    assert_bits_equal(d, z["d"])
    assert_bits_equal(e, z["e"])
    off = [o for o in range(W.shape[1]) if o - sub not in (0, 1)]
    assert np.all(W[:, off] == 0)


@pytest.mark.parametrize("sched", [bbm.BB_SCHED_STEP, bbm.BB_SCHED_PERSISTENT, bbm.BB_SCHED_GROUP])
@pytest.mark.parametrize("n,bw,tw,dt", [(700, 48, 16, "f32"), (333, 20, 7, "f64")])
def test_staged_calls_equal_reduce(n, bw, tw, dt, sched):
    """bb_pack + bb_run_pass (each pass, in order) + bb_extract == bb_reduce, and
    the working band after the first pass equals the oracle's after its first
    pass's cycles."""
    import torch
    log(f"staged n={n} bw={bw} tw={tw} {dt} sched={sched}")
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=n)
    dev = torch.device("cuda:0")
    tb = torch.from_numpy(band).to(dev)
    code = bbm.dtype_code(tb.dtype)
    info = bbm.bb_plan(n, bw, tw, code)
    work = bbm.workspace(n, bw, tw, tb.dtype, dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    tun = bbm.tuning(scheduler=sched)
    d = torch.empty(n, dtype=tb.dtype, device=dev)
    e = torch.empty(n - 1, dtype=tb.dtype, device=dev)
    bbm.bb_pack(tb.data_ptr(), tb.stride(0), n, bw, tw, code, work.data_ptr(), work.numel(), st)
    bbm.bb_run_pass(n, bw, tw, code, 0, work.data_ptr(), work.numel(), tun, st)
    W1, _ = bbm.export_band(work, n, bw, tw, tb.dtype)
    torch.cuda.synchronize()
    b0, t0 = bw, min(tw, bw - 1)
    K = [(n - 2 - R - (b0 - t0)) // b0 + 1 for R in range(max(n - (b0 - t0) - 1, 0))]
    first_pass = np.array([(0, R, k) for R in range(len(K)) for k in range(K[R])], dtype=np.int64)
    OW1 = oracle.run_cycles(band, bw, tw, first_pass)
    assert_bits_equal(W1.cpu().numpy(), OW1)
    for p in range(1, info.passes):
        bbm.bb_run_pass(n, bw, tw, code, p, work.data_ptr(), work.numel(), tun, st)
    bbm.bb_extract(work.data_ptr(), work.numel(), n, bw, tw, code, d.data_ptr(), e.data_ptr(), st)
    torch.cuda.synchronize()
    rd, re = gpu_reduce(band, bw, tw, tun)
    assert_bits_equal(d.cpu().numpy(), rd)
    assert_bits_equal(e.cpu().numpy(), re)
    # the passes in ranges (the default scheduler shares a launch within each)
    bbm.bb_pack(tb.data_ptr(), tb.stride(0), n, bw, tw, code, work.data_ptr(), work.numel(), st)
    half = info.passes // 2
    bbm.bb_run_passes(n, bw, tw, code, 0, half, work.data_ptr(), work.numel(), None, st)
    bbm.bb_run_passes(n, bw, tw, code, half, 0, work.data_ptr(), work.numel(), None, st)
    bbm.bb_run_passes(n, bw, tw, code, half, info.passes - half, work.data_ptr(), work.numel(), None, st)
    bbm.bb_extract(work.data_ptr(), work.numel(), n, bw, tw, code, d.data_ptr(), e.data_ptr(), st)
    torch.cuda.synchronize()
    assert_bits_equal(d.cpu().numpy(), rd)
    assert_bits_equal(e.cpu().numpy(), re)
