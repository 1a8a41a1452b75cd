"""GPU check of the matrix-core ceiling probe (a measurement aid beside the GEMM's
roofline, not a step of the method): every wave reports a positive cycle count and
a real-time span, and the clock they imply lies in the device's range."""
import pytest

pytestmark = pytest.mark.gpu


def test_ceiling_reports_every_wave(gpu):
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    print("[ceiling] 8 workgroups x 2048 iterations", flush=True)
    out = nv.nvfp4_mfma_ceiling(8, 2048)
    torch.cuda.synchronize()
    o = out.cpu()
    assert o.shape == (32, 2)
    assert (o[:, 0] > 0).all() and (o[:, 1] > 0).all()
    ghz = (o[:, 0].double() / (o[:, 1].double() / 100e6) / 1e9)
    assert ((ghz > 0.3) & (ghz < 4.0)).all(), ghz.tolist()
