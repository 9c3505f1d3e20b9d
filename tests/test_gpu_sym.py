"""Symmetric band -> tridiagonal on the GPU (bb_sym_reduce, through the C
ABI) against the symmetric oracle (needs a GPU).

Both sides follow the same reading of the page "A two-stage reduction on an
Apple M5 Pro", section 6, operation by operation, so d, e and the whole
working band are compared to the bit, on shapes with several sweeps per
workgroup, ragged tails, every tile size (t+1 <= 9, 17, 33, 65), one pass
and several, b' = 1 and wider targets, zero rows, few workgroups, and at the
full headline size (n = 16384, BW = 64, TW = 16) against the stored oracle
output in fp32 and on properties in fp64.
"""
import os

import numpy as np
import pytest

import band_bidiagonal_bulge_amd as bbm
import bb_inputs
import oracle
from gpu_util import assert_bits_equal, log

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

pytestmark = pytest.mark.gpu


def gpu_sym(band, bw, tw, tun=None, return_band=False):
    import torch
    dev = torch.device("cuda:0")
    tb = torch.from_numpy(np.ascontiguousarray(band)).to(dev)
    n = band.shape[0]
    work = bbm.sym_workspace(n, bw, tw, tb.dtype, dev)
    d, e = bbm.sym_reduce(tb, bw, tw, tun, work)
    torch.cuda.synchronize()
    out = [d.cpu().numpy(), e.cpu().numpy()]
    if return_band:
        ld = oracle.sym_working_ld(n, bw, tw)
        W = torch.empty((n, ld), dtype=tb.dtype, device=dev)
        bbm.bb_sym_export_band(work.data_ptr(), n, bw, tw, bbm.dtype_code(tb.dtype), W.data_ptr(),
                               torch.cuda.current_stream(dev).cuda_stream)
        torch.cuda.synchronize()
        out.append(W.cpu().numpy())
    st = bbm.bb_sym_device_status(work.data_ptr(), n, bw, tw, bbm.dtype_code(tb.dtype),
                                  torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, bbm.bb_status_str(st)
    return tuple(out)


SMALL = [
    (512, 16, 8, "f64", "normal"),
    (1000, 32, 16, "f32", "normal"),
    (777, 24, 5, "f64", "normal"),
    (300, 64, 16, "f32", "normal"),
    (257, 33, 32, "f32", "uniform"),
    (200, 65, 64, "f64", "normal"),
    (130, 10, 3, "f32", "normal"),
    (97, 9, 40, "f64", "normal"),
    (40, 39, 13, "f64", "normal"),
    (17, 16, 5, "f32", "normal"),
    (500, 48, 47, "f32", "uniform_zero_rows"),
    (64, 2, 1, "f64", "normal"),
    (3, 2, 1, "f32", "normal"),
    (1, 0, 1, "f64", "normal"),
    (500, 18, 16, "f32", "normal"),   # a b' = 2 pass (18 -> 2), then 2 -> 1
    (400, 12, 10, "f64", "normal"),   # the same in fp64 (12 -> 2 -> 1)
]


@pytest.mark.parametrize("n,bw,tw,dt,dist", SMALL)
def test_bitwise_equal_to_oracle(n, bw, tw, dt, dist):
    log(f"sym bitwise n={n} bw={bw} tw={tw} {dt} {dist}")
    band = bb_inputs.make_band(n, bw, dt, dist, seed=n + bw)
    d, e, W = gpu_sym(band, bw, tw, return_band=True)
    od, oe, OW = oracle.sym_reduce(band, bw, tw, return_band=True)
    assert_bits_equal(d, od)
    assert_bits_equal(e, oe)
    assert_bits_equal(W, OW)
    assert np.all(W[:, 2:] == 0)


@pytest.mark.parametrize("tun", [dict(max_blocks=1), dict(max_blocks=3), dict(threads_per_block=64),
                                 dict(scheduler=bbm.BB_SCHED_PERSISTENT, max_blocks=7),
                                 dict(scheduler=bbm.BB_SCHED_PERSISTENT),
                                 dict(scheduler=bbm.BB_SCHED_GROUP, group_sweeps=1),
                                 dict(scheduler=bbm.BB_SCHED_GROUP, group_sweeps=2, max_blocks=2),
                                 dict(scheduler=bbm.BB_SCHED_GROUP, group_sweeps=6, max_blocks=5)])
def test_launch_shapes(tun):
    n, bw, tw = 600, 24, 8
    log(f"sym launch shape {tun}")
    band = bb_inputs.make_band(n, bw, "f32", "normal", seed=5)
    d, e = gpu_sym(band, bw, tw, bbm.tuning(**tun))
    od, oe = oracle.sym_reduce(band, bw, tw)
    assert_bits_equal(d, od)
    assert_bits_equal(e, oe)


@pytest.mark.parametrize("n,bw,tw,dt", [(512, 16, 8, "f64"), (1000, 32, 16, "f32"), (300, 64, 16, "f32"),
                                        (257, 33, 32, "f32"), (130, 10, 3, "f32"), (500, 48, 47, "f32")])
def test_group_and_persistent_agree_to_the_bit(n, bw, tw, dt):
    log(f"sym group vs persistent n={n} bw={bw} tw={tw} {dt}")
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=2 * n + bw)
    dg, eg, Wg = gpu_sym(band, bw, tw, bbm.tuning(scheduler=bbm.BB_SCHED_GROUP), return_band=True)
    dp, ep, Wp = gpu_sym(band, bw, tw, bbm.tuning(scheduler=bbm.BB_SCHED_PERSISTENT), return_band=True)
    assert_bits_equal(Wg, Wp)
    od, oe = oracle.sym_reduce(band, bw, tw)
    assert_bits_equal(dg, od)
    assert_bits_equal(eg, oe)


@pytest.mark.parametrize("n,bw,tw,dt", [(700, 64, 16, "f32"), (500, 64, 8, "f32"), (400, 24, 8, "f64"),
                                        (300, 12, 2, "f32")])
@pytest.mark.parametrize("blocks", [0, 2])
def test_passes_in_one_launch_to_the_bit(n, bw, tw, dt, blocks):
    # the default scheduler runs consecutive group passes in one launch (at
    # most four); the result equals the oracle's and one launch per pass
    log(f"sym fused n={n} bw={bw} tw={tw} {dt} blocks={blocks}")
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=3 * n + bw)
    df, ef, Wf = gpu_sym(band, bw, tw, bbm.tuning(max_blocks=blocks), return_band=True)
    dg, eg, Wg = gpu_sym(band, bw, tw, bbm.tuning(scheduler=bbm.BB_SCHED_GROUP), return_band=True)
    assert_bits_equal(Wf, Wg)
    od, oe = oracle.sym_reduce(band, bw, tw)
    assert_bits_equal(df, od)
    assert_bits_equal(ef, oe)


def test_forced_timeout_is_reported():
    import torch
    n, bw, tw = 400, 16, 8
    log("sym forced timeout")
    band = torch.from_numpy(bb_inputs.make_band(n, bw, "f32", "normal", seed=1)).to("cuda:0")
    work = bbm.sym_workspace(n, bw, tw, band.dtype, band.device)
    for sched in (bbm.BB_SCHED_PERSISTENT, bbm.BB_SCHED_GROUP, bbm.BB_SCHED_DEFAULT):
        bbm.sym_reduce(band, bw, tw, bbm.tuning(scheduler=sched, spin_limit=1), work)
        st = bbm.bb_sym_device_status(work.data_ptr(), n, bw, tw, bbm.BB_F32,
                                      torch.cuda.current_stream().cuda_stream)
        assert st in (0, 5)   # 5: a one-poll wait expired; either way every kernel ended
    d, e = bbm.sym_reduce(band, bw, tw, None, work)       # the workspace is reusable afterwards
    torch.cuda.synchronize()
    od, oe = oracle.sym_reduce(band.cpu().numpy(), bw, tw)
    assert_bits_equal(d.cpu().numpy(), od)


def test_rejects_unsupported():
    import torch
    band = torch.zeros((100, 10), dtype=torch.float32, device="cuda:0")
    with pytest.raises(bbm.BBError):
        bbm.sym_reduce(band, 9, 4, bbm.tuning(scheduler=bbm.BB_SCHED_STEP))
    with pytest.raises(bbm.BBError):
        bbm.sym_reduce(band, 10, 4)          # ld 10 < bw + 1


def test_headline_size_equals_stored_oracle():
    # n = 16384, BW = 64, TW = 16 fp32, the shape the bench line reports: d
    # and e equal, bit for bit, the symmetric oracle's stored output
    # (tests/golden/make_golden.py --sym, oracle only), and everything off
    # the tridiagonal is exactly zero
    import hashlib
    n, bw, tw = 16384, 64, 16
    z = np.load(os.path.join(GOLDEN, "sym-n16384-bw64-tw16-f32-normal.npz"))
    band = bb_inputs.make_band(n, bw, "f32", "normal", seed=0)
    assert hashlib.sha256(band.tobytes()).hexdigest() == str(z["input_sha"])
    log("sym headline f32 vs stored oracle")
    d, e, W = gpu_sym(band, bw, tw, return_band=True)
    assert np.all(W[:, 2:] == 0)
    assert_bits_equal(d, z["d"], "d")
    assert_bits_equal(e, z["e"], "e")


def test_headline_size_properties_f64():
    # the same shape in fp64: exact zeros off the tridiagonal and the
    # Frobenius norm kept (no stored oracle output at this size in fp64)
    n, bw, tw = 16384, 64, 16
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=0)
    log("sym headline f64")
    d, e, W = gpu_sym(band, bw, tw, return_band=True)
    assert np.all(W[:, 2:] == 0)
    fro = np.sqrt(np.sum(band ** 2) * 2 - np.sum(band[:, 0] ** 2))
    t2 = np.sum(d ** 2) + 2 * np.sum(e ** 2)
    assert abs(np.sqrt(t2) - fro) <= 1e-12 * fro


def test_bitwise_at_four_thousand():
    # the page's symmetric size: n = 4096, b = 32, straight to tridiagonal
    n, bw, tw = 4096, 32, 31
    log("sym n=4096 bw=32 tw=31 f32")
    band = bb_inputs.make_band(n, bw, "f32", "normal", seed=0)
    d, e = gpu_sym(band, bw, tw)
    od, oe = oracle.sym_reduce(band, bw, tw)
    assert_bits_equal(d, od)
    assert_bits_equal(e, oe)
