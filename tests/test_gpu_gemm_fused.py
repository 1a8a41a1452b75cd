"""GPU parity of the GEMM with its fused epilogue (bias, gated residual) against the
oracle's O12, through the C ABI.

Random cases are held to the bounds derived in tests/parity.py (fused_compare),
and the residual step is checked bit for bit against its definition on the
kernel's own D1; constructed exact ties bound what the fp32 sums may round.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def dev_bf16(bits, device):
    return parity.to_device_bf16(np.ascontiguousarray(bits), device)


def quantized_operands(m, n, k, seed, device):
    x = synth.normal_bf16(m, k, seed=seed, tag=1, sigma=1.0)
    w = synth.normal_bf16(n, k, seed=seed, tag=2, sigma=0.02)
    a, aq, as_, ga = parity.run_quantize(x, None, device)
    wt, wq, ws, gw = parity.run_quantize(w, None, device)
    rq, rs, rg = oracle.quantize(x)
    rwq, rws, rgw = oracle.quantize(w)
    assert (aq == rq).all() and (wq == rwq).all() and (as_ == rs).all() and (ws == rws).all()
    return a, wt, (rq, rs, rg, rwq, rws, rgw)


def bias_vector(n, seed):
    b = synth.normal_bf16(1, n, seed=seed, tag=5, sigma=0.5)[0]
    b[0] = 0x0000
    b[1] = 0x8000
    b[2] = 0x0001   # smallest subnormal
    b[3] = 0x5F80   # 2^64
    b[4] = 0xDF80   # -2^64
    return b


@pytest.mark.parametrize("m,n,k", [(16, 16, 64), (100, 272, 192), (300, 320, 576), (513, 528, 448)])
def test_bias_and_gated_residual(gpu, m, n, k):
    check_bias_and_gated_residual(gpu, m, n, k)


def check_bias_and_gated_residual(gpu, m, n, k):
    """Bias only, and bias with gated residual, against the oracle on every element
    (n >= 16 so the planted bias and gate values fit)."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    _say(f"[fused] bias / gated residual m={m} n={n} k={k}")
    a, wt, (rq, rs, rg, rwq, rws, rgw) = quantized_operands(m, n, k, seed=m + n, device=gpu)
    m_pad = oracle.padded_rows(m)
    bias = bias_vector(n, m)
    gate = synth.normal_bf16(1, n, seed=m, tag=6, sigma=0.7)[0]
    gate[5] = 0x0000
    res = synth.normal_bf16(m_pad, n, seed=m, tag=7, sigma=0.3)
    bias_t, gate_t, res_t = dev_bf16(bias, gpu), dev_bf16(gate, gpu), dev_bf16(res, gpu)
    d1 = nv.nvfp4_gemm_bf16out_fused(a, wt, bias=bias_t)
    d = nv.nvfp4_gemm_bf16out_fused(a, wt, bias=bias_t, gate=gate_t, residual=res_t)
    torch.cuda.synchronize()
    rows = np.arange(m_pad)
    plain = oracle.gemm_rows(rq, rs, m, rg, rwq, rws, n, rgw, k, rows)
    r1, rd = oracle.gemm_rows_ex(rq, rs, m, rg, rwq, rws, n, rgw, k, rows, bias=bias, gate=gate, res=res)
    st = parity.fused_compare(parity.tensor_bits(d1), r1, plain, parity.tensor_bits(d), rd, gate)
    _say(f"[fused] {st}")
    assert st["d1_violations"] == 0 and st["d_violations"] == 0, st
    # given the GPU's own D1, the residual step is RN_bf16 of the fp32 sum
    # res + gate * D1 (the product exact): check every element
    g1 = parity.bf16_bits_to_f64(parity.tensor_bits(d1)).astype(np.float32)
    p = parity.bf16_bits_to_f64(gate).astype(np.float32)[None, :] * g1
    s = (parity.bf16_bits_to_f64(res).astype(np.float32) + p).astype(np.float64)
    want = round_f64_to_bf16(s)
    got = parity.tensor_bits(d)
    assert (got == want).all(), int((got != want).sum())


def round_f64_to_bf16(v: np.ndarray) -> np.ndarray:
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


def one_hot_operands(n, k, ga, device):
    """A: row 0 holds +1.0 at column 0, other rows zero; W: every row +1.0 at column 0;
    all block scales 1.0; so X[0, j] = g_a g_w exactly and X = 0 elsewhere."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    aq = np.zeros((16, k // 2), dtype=np.uint8)
    aq[0, 0] = 2
    wq = np.zeros((n, k // 2), dtype=np.uint8)
    wq[:, 0] = 2
    as_ = np.full(oracle.scale_bytes(16, k), 0x38, dtype=np.uint8)
    ws = np.full(oracle.scale_bytes(n, k), 0x38, dtype=np.uint8)
    a = nv.empty_nvfp4(16, k, device)
    w = nv.empty_nvfp4(n, k, device)
    a.qdata.copy_(torch.from_numpy(aq))
    a.scales.copy_(torch.from_numpy(as_))
    a.global_scale.fill_(ga)
    w.qdata.copy_(torch.from_numpy(wq))
    w.scales.copy_(torch.from_numpy(ws))
    w.global_scale.fill_(1.0)
    return a, w, (aq, as_, wq, ws)


def test_exact_ties(gpu):
    """Constructed exact ties. Bias: X = 257/256 is a bf16 midpoint and a subnormal bias
    breaks it in the exact chain. Residual: gate * D1 = 1.5 * (1 + 2^-7) is a bf16
    midpoint and a residual of -+2^-30 breaks it. The kernel sums in fp32, where
    both perturbations are below the fp32 unit, so it may round such a tie to even:
    at most one bf16 unit from the exact chain, and exact everywhere else."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    n, k = 16, 64
    a, w, (aq, as_, wq, ws) = one_hot_operands(n, k, 257.0 / 256.0, gpu)
    bias = np.array([0x0000, 0x0001, 0x8001, 0x0000] * 4, dtype=np.uint16)
    d1 = nv.nvfp4_gemm_bf16out_fused(a, w, bias=dev_bf16(bias, gpu))
    torch.cuda.synchronize()
    r1, _ = oracle.gemm_rows_ex(aq, as_, 1, 257.0 / 256.0, wq, ws, n, 1.0, k, np.arange(16), bias=bias)
    got = parity.tensor_bits(d1)
    assert (got[1:] == r1[1:]).all()
    diff = np.abs(got[0].astype(np.int32) - r1[0].astype(np.int32))
    assert (diff <= 1).all(), (got[0], r1[0])
    assert got[0, 0] == 0x3F80 and r1[0, 1] == 0x3F81

    a, w, (aq, as_, wq, ws) = one_hot_operands(n, k, 1.0 + 2.0 ** -7, gpu)
    gate = np.full(n, 0x3FC0, dtype=np.uint16)  # 1.5
    res = np.zeros((16, n), dtype=np.uint16)
    res[0, 0::3] = 0xB080  # -2^-30
    res[0, 1::3] = 0x3080  # +2^-30
    d = nv.nvfp4_gemm_bf16out_fused(a, w, gate=dev_bf16(gate, gpu), residual=dev_bf16(res, gpu))
    torch.cuda.synchronize()
    _, rd = oracle.gemm_rows_ex(aq, as_, 1, 1.0 + 2.0 ** -7, wq, ws, n, 1.0, k, np.arange(16), gate=gate, res=res)
    got = parity.tensor_bits(d)
    assert (got[1:] == rd[1:]).all()
    diff = np.abs(got[0].astype(np.int32) - rd[0].astype(np.int32))
    assert (diff <= 1).all(), (got[0], rd[0])
    assert rd[0, 0] == 0x3FC1 and got[0, 2] == 0x3FC2 and rd[0, 2] == 0x3FC2


def test_in_place_residual(gpu):
    """out is the residual tensor itself (the residual stream updated in place)."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, n, k = 300, 512, 320
    a, wt, (rq, rs, rg, rwq, rws, rgw) = quantized_operands(m, n, k, seed=77, device=gpu)
    m_pad = oracle.padded_rows(m)
    gate = synth.normal_bf16(1, n, seed=78, tag=6, sigma=0.7)[0]
    res = synth.normal_bf16(m_pad, n, seed=78, tag=7, sigma=0.3)
    res_t = dev_bf16(res, gpu)
    ref_t = nv.nvfp4_gemm_bf16out_fused(a, wt, gate=dev_bf16(gate, gpu), residual=res_t.clone())
    out = nv.nvfp4_gemm_bf16out_fused(a, wt, gate=dev_bf16(gate, gpu), residual=res_t, out=res_t)
    torch.cuda.synchronize()
    assert out.data_ptr() == res_t.data_ptr()
    assert torch.equal(res_t, ref_t)


def test_tail_quarter_tiles_fused(gpu):
    """The quarter-tile tail schedule with the fused epilogue (shape from the CU count)."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    cu = torch.cuda.get_device_properties(gpu).multi_processor_count
    tiles_n = 17
    tiles_m = (cu + cu // 16 + 16) // 17
    m, n, k = tiles_m * 256 - 96, tiles_n * 256 - 16, 320
    _say(f"[fused] quarter tail m={m} n={n} k={k} cu={cu}")
    a, wt, (rq, rs, rg, rwq, rws, rgw) = quantized_operands(m, n, k, seed=5, device=gpu)
    m_pad = oracle.padded_rows(m)
    bias = bias_vector(n, 9)
    gate = synth.normal_bf16(1, n, seed=9, tag=6, sigma=0.7)[0]
    res = synth.normal_bf16(m_pad, n, seed=9, tag=7, sigma=0.3)
    d1 = nv.nvfp4_gemm_bf16out_fused(a, wt, bias=dev_bf16(bias, gpu))
    d = nv.nvfp4_gemm_bf16out_fused(a, wt, bias=dev_bf16(bias, gpu), gate=dev_bf16(gate, gpu),
                                    residual=dev_bf16(res, gpu))
    torch.cuda.synchronize()
    rows = parity.sample_rows(m, m_pad, 600, 3)
    plain = oracle.gemm_rows(rq, rs, m, rg, rwq, rws, n, rgw, k, rows)
    r1, rd = oracle.gemm_rows_ex(rq, rs, m, rg, rwq, rws, n, rgw, k, rows, bias=bias, gate=gate, res=res)
    idx = torch.from_numpy(rows).to(gpu)
    st = parity.fused_compare(parity.tensor_bits(d1[idx]), r1, plain, parity.tensor_bits(d[idx]), rd, gate)
    _say(f"[fused] {st}")
    assert st["d1_violations"] == 0 and st["d_violations"] == 0, st


def test_canonical_fc2_fused(gpu):
    """The FC2 shape: SwiGLU producer, bias, gate and residual. The producer's bytes
    are first checked equal to the oracle's quantization, and the oracle then computes
    the fused outputs from its own bytes; 4,096 seeded rows, tile-boundary rows and
    padding rows."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    w = synth.FC2
    _say("[fused] canonical FC2")
    gate_in, up_in = w.activations()
    a, aq, as_, ga = parity.run_quantize(gate_in, up_in, gpu)
    rq, rs, rg = oracle.quantize(gate_in, up_in)
    assert (aq == rq).all() and (as_ == rs).all() and ga == rg, "activation bytes differ from the oracle"
    del gate_in, up_in, aq, as_
    W = w.weight()
    wt, wq, ws, gw = parity.run_quantize(W, None, gpu)
    rwq, rws, rgw = oracle.quantize(W)
    assert (wq == rwq).all() and (ws == rws).all() and gw == rgw, "weight bytes differ from the oracle"
    del W, wq, ws
    bias = bias_vector(w.n, 11)
    gate = synth.normal_bf16(1, w.n, seed=11, tag=6, sigma=0.7)[0]
    res = synth.normal_bf16(w.m_pad, w.n, seed=11, tag=7, sigma=0.3)
    d1 = nv.nvfp4_gemm_bf16out_fused(a, wt, bias=dev_bf16(bias, gpu))
    d = nv.nvfp4_gemm_bf16out_fused(a, wt, bias=dev_bf16(bias, gpu), gate=dev_bf16(gate, gpu),
                                    residual=dev_bf16(res, gpu))
    torch.cuda.synchronize()
    rows = parity.sample_rows(w.m, w.m_pad, parity.PARITY_ROWS, 12)
    _say(f"[fused] canonical FC2: oracle on {rows.size} rows")
    plain = oracle.gemm_rows(rq, rs, w.m, rg, rwq, rws, w.n, rgw, w.k, rows)
    r1, rd = oracle.gemm_rows_ex(rq, rs, w.m, rg, rwq, rws, w.n, rgw, w.k, rows, bias=bias, gate=gate, res=res)
    idx = torch.from_numpy(rows).to(gpu)
    st = parity.fused_compare(parity.tensor_bits(d1[idx]), r1, plain, parity.tensor_bits(d[idx]), rd, gate)
    _say(f"[fused] {st}")
    assert st["d1_violations"] == 0 and st["d_violations"] == 0, st
    assert st["checked"] >= parity.PARITY_ROWS * w.n
