"""GPU parity of the modulated plain producer (nvfp4_quantize_modulate) against the
oracle's O13 + O3-O8, through the C ABI: QDATA, scale buffer and global scale
bit-exact, padding included.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_mod(x_bits, sc, sh, device, m=None):
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    x = parity.to_device_bf16(x_bits, device)
    t = nv.nvfp4_quantize_modulate(x, parity.to_device_bf16(sc, device), parity.to_device_bf16(sh, device), rows=m)
    torch.cuda.synchronize(device)
    return t.qdata.cpu().numpy(), t.scales.cpu().numpy(), float(t.global_scale.item())


def check_mod(x_bits, sc, sh, device, what, m=None):
    _say(f"[producer-mod] {what}: shape {x_bits.shape} m={m}")
    qd, scl, g = run_mod(x_bits, sc, sh, device, m=m)
    rq, rs, rg = oracle.quantize_modulate(x_bits, sc, sh, m=m)
    assert np.float32(g).view(np.uint32) == np.float32(rg).view(np.uint32), f"{what}: g {g!r} != {rg!r}"
    nq = int((qd != rq).sum())
    ns = int((scl != rs).sum())
    assert nq == 0 and ns == 0, f"{what}: {nq} QDATA bytes and {ns} scale bytes differ"


def vectors(k, seed, s_sigma=0.3, b_sigma=0.5):
    sc = synth.normal_bf16(1, k, seed=seed, tag=21, sigma=s_sigma)[0]
    sh = synth.normal_bf16(1, k, seed=seed, tag=22, sigma=b_sigma)[0]
    return sc, sh


@pytest.mark.parametrize("m,k", [(1, 64), (15, 64), (17, 192), (130, 320), (255, 1024), (300, 576)])
def test_edge_shapes(gpu, m, k):
    """Ragged rows (padding must stay zero although the shift is not), widths that do
    not fill a work item."""
    x = synth.normal_bf16(m, k, seed=m + 500, tag=1, sigma=1.0)
    sc, sh = vectors(k, m)
    check_mod(x, sc, sh, gpu, f"m={m} k={k}")


def test_special_vectors(gpu):
    """scale -1 (y = shift), scale 0 and shift 0 (y = x), tiny and huge magnitudes,
    subnormal results, signed zeros."""
    m, k = 64, 256
    x = synth.normal_bf16(m, k, seed=3, tag=1, sigma=1.0)
    x[5, :] = 0x8000
    x[6, :64] = 0x0001
    sc, sh = vectors(k, 3)
    sc[:16] = 0xBF80   # -1
    sc[16:32] = 0x0000
    sh[16:32] = 0x0000
    sc[32:48] = 0x3380  # 2^-24: 1 + s rounds to 1
    sh[48:64] = 0x0001  # smallest subnormal shift
    sc[64:80] = 0x4700  # 32768
    check_mod(x, sc, sh, gpu, "special vectors")
    y = synth.normal_bf16(m, k, seed=4, tag=1, sigma=1e-30)
    check_mod(y, np.zeros(k, np.uint16), np.zeros(k, np.uint16), gpu, "tiny x, identity modulation")


def test_strided_rows(gpu):
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, k, ld = 70, 320, 384
    base = synth.normal_bf16(m, ld, seed=8, tag=1, sigma=1.0)
    sc, sh = vectors(k, 8)
    t = parity.to_device_bf16(base, gpu)[:, :k]
    out = nv.nvfp4_quantize_modulate(t, parity.to_device_bf16(sc, gpu), parity.to_device_bf16(sh, gpu))
    torch.cuda.synchronize(gpu)
    rq, rs, rg = oracle.quantize_modulate(np.ascontiguousarray(base[:, :k]), sc, sh)
    assert (out.qdata.cpu().numpy() == rq).all() and (out.scales.cpu().numpy() == rs).all()
    assert float(out.global_scale.item()) == rg


@pytest.mark.parametrize("name", ["qkv", "fc1"])
def test_full_size_inputs(gpu, name):
    """The QKV and FC1 input at full size (M = 37,810, K = 5,376) with seeded
    modulation vectors."""
    w = synth.BY_NAME[name]
    x = w.activations()[0]
    sc, sh = vectors(w.k, 40 + len(name))
    check_mod(x, sc, sh, gpu, name)
