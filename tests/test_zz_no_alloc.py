"""bb_reduce_noalloc (the entry point that allocates nothing; its workspace is
the library's fixed per-GPU array) against bb_reduce with a caller workspace:
bit patterns equal, on consecutive calls each smaller than the one before
(the array keeps the previous call's contents; the third has a pass on
windowed ring rows), and the status word it hands back; shapes above the
array's size are refused."""
import numpy as np
import pytest

import band_bidiagonal_bulge_amd as bbm
import bb_inputs
from gpu_util import assert_bits_equal, log

pytestmark = pytest.mark.gpu

CALLS = [(16384, 64, 16, "f32"), (4096, 32, 16, "f32"), (900, 64, 31, "f32"), (777, 20, 7, "f64")]


def _noalloc(tb, bw, tw, status):
    import torch
    n = tb.shape[0]
    d = torch.full((n,), float("nan"), dtype=tb.dtype, device=tb.device)
    e = torch.full((max(n - 1, 0),), float("nan"), dtype=tb.dtype, device=tb.device)
    status.fill_(12345)
    bbm.bb_reduce_noalloc(tb.data_ptr(), tb.stride(0), n, bw, tw, bbm.dtype_code(tb.dtype), d.data_ptr(),
                          e.data_ptr() if n > 1 else 0, status.data_ptr(), None,
                          torch.cuda.current_stream(tb.device).cuda_stream)
    torch.cuda.synchronize()
    return d.cpu().numpy(), e.cpu().numpy(), int(status.item())


def test_noalloc_equals_bb_reduce_on_consecutive_calls():
    import torch
    dev = torch.device("cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for (n, bw, tw, dt) in CALLS:
        log(f"bb_reduce_noalloc n={n} bw={bw} tw={tw} {dt}")
        tb = torch.from_numpy(bb_inputs.make_band(n, bw, dt, "normal", seed=n)).to(dev)
        dn, en, st = _noalloc(tb, bw, tw, status)
        assert st == 0
        d, e = bbm.reduce(tb, bw, tw, check=True)
        torch.cuda.synchronize()
        assert_bits_equal(dn, d.cpu().numpy(), f"d n={n}")
        assert_bits_equal(en, e.cpu().numpy(), f"e n={n}")
        assert np.all(np.isfinite(dn)) and np.all(np.isfinite(en))


def test_noalloc_refuses_shapes_above_its_array():
    import torch
    x = torch.zeros(8, dtype=torch.float64, device="cuda:0")
    assert bbm.bb_workspace_bytes(32768, 128, 32, bbm.BB_F64) > bbm.BB_NOALLOC_SCRATCH_BYTES
    with pytest.raises(bbm.BBError) as ex:
        bbm.bb_reduce_noalloc(x.data_ptr(), 129, 32768, 128, 32, bbm.BB_F64, x.data_ptr(), x.data_ptr(), 0, None, 0)
    assert ex.value.status == bbm.BB_ERR_WORKSPACE
