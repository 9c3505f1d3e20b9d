"""Half-precision band -> bidiagonal on the GPU (dtype BB_F16, through the C
ABI) against the fp16 oracle, and the accuracy study of the page
"Accelerating Bidiagonalization of Banded Matrices through Memory-Aware
Bulge-Chasing on GPUs" (known singular values, reduction in FP64 / FP32 /
FP16, singular values in fp64) on a small scale (needs a GPU).
"""
import numpy as np
import pytest

import band_bidiagonal_bulge_amd as bbm
import bb_inputs
import oracle
from gpu_util import assert_bits_equal, gpu_reduce, log

pytestmark = pytest.mark.gpu

SHAPES = [(512, 16, 8), (300, 64, 16), (257, 33, 32), (130, 10, 3), (97, 9, 40), (40, 39, 13), (17, 16, 5),
          (600, 32, 16), (200, 65, 64)]


@pytest.mark.parametrize("n,bw,tw", SHAPES)
def test_bitwise_equal_to_fp16_oracle(n, bw, tw):
    log(f"f16 bitwise n={n} bw={bw} tw={tw}")
    band = bb_inputs.make_band(n, bw, "f16", "normal", seed=n + bw)
    d, e, W, sub = gpu_reduce(band, bw, tw, return_band=True)
    od, oe, OW, osub = oracle.reduce(band, bw, tw, return_band=True)
    assert d.dtype == np.float16 and sub == osub
    assert_bits_equal(d.view(np.uint16), od.view(np.uint16))
    assert_bits_equal(e.view(np.uint16), oe.view(np.uint16))
    assert_bits_equal(W.view(np.uint16), OW.view(np.uint16))


def test_launch_shapes_and_zero_rows():
    n, bw, tw = 400, 24, 8
    band = bb_inputs.make_band(n, bw, "f16", "uniform_zero_rows", seed=3)
    od, oe = oracle.reduce(band, bw, tw)
    for tun in (dict(max_blocks=1), dict(max_blocks=5, threads_per_block=64),
                dict(scheduler=bbm.BB_SCHED_PERSISTENT), dict(scheduler=bbm.BB_SCHED_GROUP, group_sweeps=3),
                dict(scheduler=bbm.BB_SCHED_GROUP, group_sweeps=6, max_blocks=2)):
        log(f"f16 launch shape {tun}")
        d, e = gpu_reduce(band, bw, tw, bbm.tuning(**tun))
        assert_bits_equal(d.view(np.uint16), od.view(np.uint16))
        assert_bits_equal(e.view(np.uint16), oe.view(np.uint16))


@pytest.mark.parametrize("n,bw,tw", [(600, 32, 16), (300, 64, 16), (512, 16, 8)])
def test_group_and_persistent_agree_to_the_bit(n, bw, tw):
    band = bb_inputs.make_band(n, bw, "f16", "normal", seed=n)
    log(f"f16 group vs persistent n={n} bw={bw} tw={tw}")
    dg, eg, Wg, _ = gpu_reduce(band, bw, tw, bbm.tuning(scheduler=bbm.BB_SCHED_GROUP), return_band=True)
    dp, ep, Wp, _ = gpu_reduce(band, bw, tw, bbm.tuning(scheduler=bbm.BB_SCHED_PERSISTENT), return_band=True)
    assert_bits_equal(Wg.view(np.uint16), Wp.view(np.uint16))


def test_unsupported_combinations():
    import torch
    band = torch.zeros((64, 9), dtype=torch.float16, device="cuda:0")
    with pytest.raises(bbm.BBError):
        bbm.reduce(band, 8, 4, bbm.tuning(scheduler=bbm.BB_SCHED_STEP))
    with pytest.raises(bbm.BBError):
        bbm.sym_reduce(band, 8, 4)
    d = torch.ones(8, dtype=torch.float16, device="cuda:0")
    with pytest.raises((bbm.BBError, TypeError)):
        bbm.svals(d, d[:7])


def test_headline_shape_in_half_precision():
    # n = 16384, BW = 64, TW = 16 in binary16, the shape the bench line
    # reports: d and e equal, bit for bit, the emulated-binary16 oracle's
    # stored output (tests/golden/make_golden.py --f16, oracle only), and
    # everything off the bidiagonal is exactly zero
    import hashlib
    import os
    n, bw, tw = 16384, 64, 16
    z = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                             "n16384-bw64-tw16-f16-normal.npz"))
    band = bb_inputs.make_band(n, bw, "f16", "normal", seed=0)
    assert hashlib.sha256(band.tobytes()).hexdigest() == str(z["input_sha"])
    log("f16 headline shape vs stored oracle")
    d, e, W, sub = gpu_reduce(band, bw, tw, return_band=True)
    off = [o for o in range(W.shape[1]) if o - sub not in (0, 1)]
    assert np.all(W[:, off] == 0)
    assert_bits_equal(d.view(np.uint16), z["d"].view(np.uint16), "d")
    assert_bits_equal(e.view(np.uint16), z["e"].view(np.uint16), "e")


def test_accuracy_study_small():
    # each precision's relative singular-value error on known spectra, with
    # the fp16 and fp32 GPU bits equal to the oracle's on the first instance
    import torch
    n, bw, tw = 192, 16, 8
    worst = {}
    for spectrum in bb_inputs.SPECTRA:
        for seed in range(2):
            band64, sigma = bb_inputs.known_spectrum_band(n, bw, spectrum, seed=seed)
            for dt in ("f64", "f32", "f16"):
                band = band64.astype(bb_inputs.np_dtype(dt))
                log(f"accuracy {spectrum} seed={seed} {dt}")
                d, e = gpu_reduce(band, bw, tw)
                if seed == 0:
                    od, oe = oracle.reduce(band, bw, tw)
                    assert_bits_equal(d, od)
                    assert_bits_equal(e, oe)
                td = torch.from_numpy(d.astype(np.float64)).to("cuda:0")
                te = torch.from_numpy(e.astype(np.float64)).to("cuda:0")
                sv = bbm.svals(td, te).cpu().numpy()
                rel = np.linalg.norm(sv - sigma) / np.linalg.norm(sigma)
                worst[dt] = max(worst.get(dt, 0.0), rel)
    log(f"accuracy worst relative errors: {worst}")
    assert worst["f64"] < 1e-13 and worst["f32"] < 1e-5 and worst["f16"] < 5e-2
    assert worst["f64"] < worst["f32"] < worst["f16"]
