"""The bandwidth probes' results (needs a GPU): z = x + y and B = A + A^T
against torch on the same device, including ragged sizes and repeated
operations (the result does not depend on the repetition count)."""
import pytest

import band_bidiagonal_bulge_amd as bbm
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,reps", [(4, 1), (1 << 20, 1), ((1 << 20) + 12, 3), (3 << 18, 7)])
def test_stream_probe(n, reps):
    import torch
    log(f"stream probe n={n} reps={reps}")
    g = torch.Generator(device="cpu").manual_seed(n)
    x = torch.randn(n, generator=g).to("cuda:0")
    y = torch.randn(n, generator=g).to("cuda:0")
    z = torch.full((n,), float("nan"), device="cuda:0")
    bbm.bb_probe_stream(x.data_ptr(), y.data_ptr(), z.data_ptr(), n, reps, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(z, x + y)


@pytest.mark.parametrize("m,reps", [(1, 1), (63, 2), (64, 1), (130, 3), (1000, 5)])
def test_transpose_add_probe(m, reps):
    import torch
    log(f"transpose-add probe m={m} reps={reps}")
    g = torch.Generator(device="cpu").manual_seed(m)
    a = torch.randn(m, m, generator=g).to("cuda:0")
    b = torch.full_like(a, float("nan"))
    bbm.bb_probe_transpose_add(a.data_ptr(), b.data_ptr(), m, reps, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(b, a + a.t().contiguous())


def test_probe_argument_checks():
    import torch
    x = torch.zeros(8, device="cuda:0")
    p = x.data_ptr()
    with pytest.raises(bbm.BBError):
        bbm.bb_probe_stream(p, p, p + 32, 6, 1, 0)  # not a multiple of 4
    with pytest.raises(bbm.BBError):
        bbm.bb_probe_stream(p, p, p, 4, 0, 0)  # no repetition
    with pytest.raises(bbm.BBError):
        bbm.bb_probe_transpose_add(p, p, 2, 1, 0)  # in place
    with pytest.raises(bbm.BBError):
        bbm.bb_probe_transpose_add(p, p + 16, -1, 1, 0)


@pytest.mark.parametrize("m", [17, 33])
def test_norm_probe_runs(m):
    import torch
    log(f"norm probe m={m}")
    x = torch.rand(64, device="cuda:0")
    out = torch.zeros(64, device="cuda:0")
    clk = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    for mode in (0, 1):
        bbm.bb_probe_norm_clocks(m, mode, 100, x.data_ptr(), out.data_ptr(), clk.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert clk.item() > 0
        # one norm alone: both ways sum the same squares to within rounding
        ref = float((x[1:m].double() ** 2).sum())
        assert abs(out[0].item() / 100 - ref) <= 1e-4 * ref
    with pytest.raises(bbm.BBError):
        bbm.bb_probe_norm_clocks(16, 0, 1, x.data_ptr(), out.data_ptr(), clk.data_ptr(), 0)
