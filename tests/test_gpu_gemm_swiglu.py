"""GPU parity of the SwiGLU-pair GEMM (nvfp4_gemm_swiglu_pair) against the oracle's
O14, and of the chain it enables: FC1 emits the amax, the single-read FC2 producer
takes it, and its bytes equal those of the two-pass producer.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def bf16_round_f64(v):
    """numpy RNE of exact float64 values to bf16 bits (finite)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(np.where(a == 0, 1.0, a))
    lead = np.maximum(e - 1, -126)
    q = np.ldexp(1.0, lead - 7)
    r = (np.rint(a / q) * q).astype(np.float32)
    bits = (r.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.signbit(v) & (a != 0), bits | 0x8000, bits)
    return np.where(a == 0, 0, bits).astype(np.uint16)


def swiglu_abs_max(gate_bits, up_bits):
    """max |RN_bf16(silu_bf16(gate) * up)| with the oracle's silu table; the product of
    two bf16 values is exact in float64."""
    tab = oracle.silu_table()
    s = parity.bf16_bits_to_f64(tab[gate_bits])
    u = parity.bf16_bits_to_f64(up_bits)
    y = bf16_round_f64(s * u)
    return float(np.abs(parity.bf16_bits_to_f64(y)).max()) if y.size else 0.0


def make_operands(m, n_half, k, seed, device):
    x = synth.normal_bf16(m, k, seed=seed, tag=1, sigma=1.0)
    wg = synth.normal_bf16(n_half, k, seed=seed, tag=2, sigma=0.05)
    wu = synth.normal_bf16(n_half, k, seed=seed, tag=3, sigma=0.05)
    w = oracle.interleave_swiglu_rows(wg, wu)
    a, aq, as_, ga = parity.run_quantize(x, None, device)
    wt, wq, ws, gw = parity.run_quantize(w, None, device)
    rq, rs, rg = oracle.quantize(x)
    rwq, rws, rgw = oracle.quantize(w)
    assert (aq == rq).all() and (wq == rwq).all() and (as_ == rs).all() and (ws == rws).all()
    return a, wt, (rq, rs, rg, rwq, rws, rgw)


def run_pair(a, wt, bias, device):
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    amax = torch.zeros(1, dtype=torch.float32, device=device)
    b = None if bias is None else parity.to_device_bf16(bias, device)
    g, u = nv.nvfp4_gemm_swiglu_pair(a, wt, bias=b, amax=amax)
    torch.cuda.synchronize(device)
    return g, u, float(amax.item())


@pytest.mark.parametrize("m,n_half,k", [(16, 8, 64), (100, 136, 192), (300, 256, 320), (513, 264, 448)])
def test_pair_against_oracle(gpu, m, n_half, k):
    check_pair(gpu, m, n_half, k)


def check_pair(gpu, m, n_half, k):
    """Gate and up with bias against the oracle on every element, and the emitted amax."""
    _say(f"[swiglu-pair] m={m} n_half={n_half} k={k}")
    a, wt, (rq, rs, rg, rwq, rws, rgw) = make_operands(m, n_half, k, m + n_half, gpu)
    bias = synth.normal_bf16(1, 2 * n_half, seed=m, tag=5, sigma=0.2)[0]
    g, u, amax = run_pair(a, wt, bias, gpu)
    m_pad = oracle.padded_rows(m)
    rows = np.arange(m_pad)
    rg0, ru0, _ = oracle.gemm_swiglu_rows(rq, rs, m, rg, rwq, rws, n_half, rgw, k, rows)
    rgt, rut, rymax = oracle.gemm_swiglu_rows(rq, rs, m, rg, rwq, rws, n_half, rgw, k, rows, bias=bias)
    gb, ub = parity.tensor_bits(g), parity.tensor_bits(u)
    for name, got, ref, plain in (("gate", gb, rgt, rg0), ("up", ub, rut, ru0)):
        st = parity.fused_compare(got, ref, plain)
        assert st["d1_violations"] == 0, (name, st)
    # the emitted amax is exactly max |y| of the kernel's own gate and up (logical rows)
    want = swiglu_abs_max(gb[:m], ub[:m])
    assert np.float32(amax) == np.float32(want), (amax, want)
    # and close to the oracle's (gate and up within the GEMM tolerance)
    ref_amax = float(rymax[:m].max())
    assert abs(amax - ref_amax) <= 2.0 ** -6 * ref_amax


def test_amax_accumulates_and_excludes_padding(gpu):
    """The kernel folds into the caller's value (a larger start survives) and ignores
    rows past amax_rows."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, n_half, k = 40, 64, 128
    a, wt, _ = make_operands(m, n_half, k, 3, gpu)
    bias = np.full(2 * n_half, 0x4300, np.uint16)  # 128: padding rows would give y ~ 128^2
    b = parity.to_device_bf16(bias, gpu)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    g, u = nv.nvfp4_gemm_swiglu_pair(a, wt, bias=b, amax=amax)
    torch.cuda.synchronize(gpu)
    want = swiglu_abs_max(parity.tensor_bits(g)[:m], parity.tensor_bits(u)[:m])
    assert float(amax.item()) == want
    big = torch.full((1,), 1e30, dtype=torch.float32, device=gpu)
    nv.nvfp4_gemm_swiglu_pair(a, wt, bias=b, amax=big)
    torch.cuda.synchronize(gpu)
    assert float(big.item()) == np.float32(1e30)


def test_pair_without_amax(gpu):
    """With no amax pointer the gate and up outputs are the same bytes."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, n_half, k = 300, 256, 320
    a, wt, _ = make_operands(m, n_half, k, 13, gpu)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    g1, u1 = nv.nvfp4_gemm_swiglu_pair(a, wt, amax=amax)
    g0, u0 = nv.nvfp4_gemm_swiglu_pair(a, wt)
    torch.cuda.synchronize(gpu)
    assert torch.equal(g0, g1) and torch.equal(u0, u1)
    assert float(amax.item()) > 0.0


@pytest.mark.parametrize("log2_scale", [-60, -66, -72, 0, 63, 66])
def test_amax_extreme_magnitudes(gpu, log2_scale):
    """The amax stays exactly max |y| of the kernel's own outputs when the outputs are
    scaled by a power of two (through the activation's global scale): products in the
    bf16 subnormal range or underflowing to zero (where the register screen's threshold
    is 0 and every half is scanned exactly), and products that overflow bf16 to inf."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, n_half, k = 300, 256, 320
    _say(f"[swiglu-pair] outputs scaled by 2^{log2_scale}")
    a, wt, _ = make_operands(m, n_half, k, 11, gpu)
    a.global_scale.mul_(2.0 ** log2_scale)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    g, u = nv.nvfp4_gemm_swiglu_pair(a, wt, amax=amax)
    torch.cuda.synchronize(gpu)
    gb, ub = parity.tensor_bits(g), parity.tensor_bits(u)
    with np.errstate(over="ignore", invalid="ignore"):
        want = swiglu_abs_max(gb[:m], ub[:m])
    got = float(amax.item())
    assert np.float32(got) == np.float32(want), (got, want)
    if log2_scale == 66:
        assert np.isinf(got)
    if log2_scale == -66:
        assert 0.0 < got < 2.0 ** -120


def test_chain_small(gpu):
    """FC1 pair GEMM -> amax -> single-read producer equals the two-pass producer and
    the oracle, byte for byte."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, n_half, k = 300, 512, 320
    a, wt, _ = make_operands(m, n_half, k, 9, gpu)
    g, u, _ = run_pair(a, wt, None, gpu)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    g, u = nv.nvfp4_gemm_swiglu_pair(a, wt, amax=amax)
    one = nv.nvfp4_quantize_swiglu_amax(g[:m], u[:m], amax)
    two = nv.nvfp4_quantize_swiglu(g[:m], u[:m])
    torch.cuda.synchronize(gpu)
    assert torch.equal(one.qdata, two.qdata) and torch.equal(one.scales, two.scales)
    assert torch.equal(one.global_scale, two.global_scale)
    rq, rs, rg = oracle.quantize(parity.tensor_bits(g)[:m], parity.tensor_bits(u)[:m])
    assert (one.qdata.cpu().numpy() == rq).all() and (one.scales.cpu().numpy() == rs).all()


def test_fc1_full_size_chain(gpu):
    """The FC1 shape (M = 37,810, 2 x 14,336 outputs, K = 5,376): sampled rows against
    the oracle, the emitted amax against max |y| of the whole output, and the
    single-read FC2 producer against the two-pass one."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    w = synth.BY_NAME["fc1"]
    _say("[swiglu-pair] FC1 full size")
    x = w.activations()[0]
    W = w.weight()
    n_half = w.n // 2
    Wi = oracle.interleave_swiglu_rows(W[:n_half], W[n_half:])
    del W
    a, aq, as_, ga = parity.run_quantize(x, None, gpu)
    wt, wq, ws, gw = parity.run_quantize(Wi, None, gpu)
    del Wi, x
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    g, u = nv.nvfp4_gemm_swiglu_pair(a, wt, amax=amax)
    torch.cuda.synchronize(gpu)
    rows = parity.sample_rows(w.m, w.m_pad, 48, 21)
    rgt, rut, _ = oracle.gemm_swiglu_rows(aq, as_, w.m, ga, wq, ws, n_half, gw, w.k, rows)
    idx = torch.from_numpy(rows).to(gpu)
    for name, got, ref in (("gate", parity.tensor_bits(g[idx]), rgt), ("up", parity.tensor_bits(u[idx]), rut)):
        st = parity.gemm_compare(got, ref)
        assert st["violations"] == 0 and st["rel_fro"] <= parity.REL_FRO_TOL, (name, st)
    # max |y| over the whole output, on the GPU with the library's pinned silu table
    sg = nv.nvfp4_silu_bf16(g[: w.m].contiguous().view(torch.int16)).view(torch.bfloat16)
    ymax = (sg.float() * u[: w.m].float()).bfloat16().abs().max().float()
    del sg
    assert float(amax.item()) == float(ymax.item())
    one = nv.nvfp4_quantize_swiglu_amax(g[: w.m], u[: w.m], amax)
    two = nv.nvfp4_quantize_swiglu(g[: w.m], u[: w.m])
    torch.cuda.synchronize(gpu)
    assert torch.equal(one.qdata, two.qdata) and torch.equal(one.scales, two.scales)
    assert torch.equal(one.global_scale, two.global_scale)
