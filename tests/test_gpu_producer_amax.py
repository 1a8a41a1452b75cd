"""GPU parity of the single-read producer (caller-supplied amax) against the oracle's
O11, through the C ABI: QDATA, scale buffer and global scale bit-exact, padding
included.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def true_amax(x_bits, up_bits, m=None) -> float:
    _, _, _, y = oracle.quantize(x_bits, up_bits, m=m, return_y=True)
    return float(np.abs(oracle.bf16_bits_to_f32(y).astype(np.float64)).max()) if y.size else 0.0


def run_amax(x_bits, up_bits, amax, device, m=None):
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    x = parity.to_device_bf16(x_bits, device)
    a = torch.tensor([amax], dtype=torch.float32, device=device)
    if up_bits is not None:
        u = parity.to_device_bf16(up_bits, device)
        t = nv.nvfp4_quantize_swiglu_amax(x, u, a, m=m)
    else:
        t = nv.nvfp4_quantize_amax(x, a, rows=m)
    torch.cuda.synchronize(device)
    return t.qdata.cpu().numpy(), t.scales.cpu().numpy(), float(t.global_scale.item())


def check_amax(x_bits, up_bits, amax, device, what, m=None):
    _say(f"[producer-amax] {what}: shape {x_bits.shape} m={m} amax={amax!r}")
    qd, sc, g = run_amax(x_bits, up_bits, amax, device, m=m)
    rq, rs, rg = oracle.quantize_amax(x_bits, up_bits, amax, m=m)
    assert np.float32(g).view(np.uint32) == np.float32(rg).view(np.uint32), f"{what}: g {g!r} != {rg!r}"
    nq = int((qd != rq).sum())
    ns = int((sc != rs).sum())
    assert nq == 0 and ns == 0, f"{what}: {nq} QDATA bytes and {ns} scale bytes differ"


def test_tiny_true_amax(gpu):
    w = synth.TINY
    gate, up = w.activations()
    check_amax(gate, up, true_amax(gate, up), gpu, "tiny swiglu")
    x = w.weight()
    check_amax(x, None, true_amax(x, None), gpu, "tiny weight")


@pytest.mark.parametrize("factor", [1.0, 1.25, 64.0, 0.5, 1e-4])
def test_amax_above_and_below(gpu, factor):
    """Above the true maximum (coarser global scale) and below it (saturating blocks)."""
    gate = synth.normal_bf16(300, 576, seed=21, tag=1, sigma=1.0)
    up = synth.normal_bf16(300, 576, seed=21, tag=2, sigma=1.0)
    check_amax(gate, up, true_amax(gate, up) * factor, gpu, f"swiglu x{factor}")
    check_amax(gate, None, true_amax(gate, None) * factor, gpu, f"plain x{factor}")


@pytest.mark.parametrize("amax", [0.0, -2.0, float("nan")])
def test_degenerate_amax(gpu, amax):
    gate = synth.normal_bf16(40, 128, seed=22, tag=1, sigma=1.0)
    up = synth.normal_bf16(40, 128, seed=22, tag=2, sigma=1.0)
    check_amax(gate, up, amax, gpu, "degenerate")


@pytest.mark.parametrize("m,k", [(1, 64), (17, 192), (130, 320), (255, 1024)])
def test_edge_shapes(gpu, m, k):
    gate = synth.normal_bf16(m, k, seed=m + 1000, tag=1, sigma=1.0)
    up = synth.normal_bf16(m, k, seed=m + 1000, tag=2, sigma=1.0)
    check_amax(gate, up, true_amax(gate, up), gpu, f"m={m} k={k}")


def test_empty_rows(gpu):
    """m = 0: only g (from the given amax) is written."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    k = 128
    x = torch.zeros((1, k), dtype=torch.bfloat16, device=gpu)
    a = torch.tensor([5376.0], dtype=torch.float32, device=gpu)
    t = nv.nvfp4_quantize_swiglu_amax(x, x, a, m=0)
    torch.cuda.synchronize(gpu)
    assert float(t.global_scale.item()) == 2.0


def test_strided_inputs(gpu):
    """Row strides larger than k, different for gate and up (the FC1 pair GEMM's gate
    and up outputs are read this way when a caller slices a wider buffer)."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, k = 150, 448
    gate_full = synth.normal_bf16(m, k + 64, seed=23, tag=1, sigma=1.0)
    up_full = synth.normal_bf16(m, k + 192, seed=23, tag=2, sigma=1.0)
    gate, up = np.ascontiguousarray(gate_full[:, :k]), np.ascontiguousarray(up_full[:, :k])
    amax = true_amax(gate, up)
    _say(f"[producer-amax] strided m={m} k={k}")
    g_t = parity.to_device_bf16(gate_full, gpu)[:, :k]
    u_t = parity.to_device_bf16(up_full, gpu)[:, :k]
    a = torch.tensor([amax], dtype=torch.float32, device=gpu)
    t = nv.nvfp4_quantize_swiglu_amax(g_t, u_t, a)
    x_t = parity.to_device_bf16(gate_full, gpu)[:, :k]
    ax = torch.tensor([true_amax(gate, None)], dtype=torch.float32, device=gpu)
    t2 = nv.nvfp4_quantize_amax(x_t, ax)
    torch.cuda.synchronize(gpu)
    rq, rs, rg = oracle.quantize_amax(gate, up, amax)
    assert (t.qdata.cpu().numpy() == rq).all() and (t.scales.cpu().numpy() == rs).all()
    assert np.float32(t.global_scale.item()) == np.float32(rg)
    rq2, rs2, rg2 = oracle.quantize_amax(gate, None, true_amax(gate, None))
    assert (t2.qdata.cpu().numpy() == rq2).all() and (t2.scales.cpu().numpy() == rs2).all()
    assert np.float32(t2.global_scale.item()) == np.float32(rg2)


def test_mid_and_outliers(gpu):
    w = synth.BY_NAME["mid_fc2_slice"]
    gate, up = w.activations()
    check_amax(gate, up, true_amax(gate, up), gpu, "mid fc2 slice")


def test_canonical_fc2(gpu):
    """The full FC2 activation with its true amax: identical to the two-pass producer's
    oracle result, element by element."""
    w = synth.FC2
    gate, up = w.activations()
    check_amax(gate, up, true_amax(gate, up), gpu, "canonical fc2")
