"""Pins for the oracle's block-scaled GEMM (step O10): E2M1 x E2M1 with vector-16
UE4M3 scales and FP32 global scales, BF16 output ("FC2 NVFP4 Scheduling Results",
section "Canonical Operation"). The oracle evaluates the sum exactly and rounds
once; these tests check it against fp64 dequantize-then-matmul and against
special cases that reduce to a gather, a row sum and a transpose.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact


def round_f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """Independent numpy RNE of float64 values to bf16 bits (finite inputs)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(np.where(a == 0, 1.0, a))
    lead = np.maximum(e - 1, -126)
    q = np.ldexp(1.0, lead - 7)
    n = np.rint(a / q)
    r = (n * q).astype(np.float32)
    bits = (r.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(v < 0, bits | 0x8000, bits)
    return np.where(a == 0, 0, bits).astype(np.uint16)


def boundary_distance(v: np.ndarray) -> np.ndarray:
    """Relative distance of |v| to the nearest bf16 rounding boundary."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(a == 0, 1.0, a))
    q = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    fr = a / q - np.floor(a / q)
    return np.where(a == 0, 1.0, np.abs(fr - 0.5) * q / np.where(a == 0, 1.0, a))


def dequant(qdata: np.ndarray, scales: np.ndarray, rows: int, k: int, g: float) -> np.ndarray:
    """fp64 dequantization written from the bit-level format definitions."""
    lo = qdata & 15
    hi = qdata >> 4
    codes = np.empty((qdata.shape[0], k), dtype=np.uint8)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    e2m1 = np.array([float(exact.e2m1_bits_value(c)) for c in range(16)])
    ue4m3 = np.array([float(exact.ue4m3_bits_value(b)) for b in range(128)] + [0.0] * 128)
    cpad = oracle.scale_cols(k)
    r = np.arange(qdata.shape[0])[:, None]
    c = np.arange(k // 16)[None, :]
    off = ((r >> 7) * (cpad // 4) + (c >> 2)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 3)
    s = ue4m3[scales[off]]
    return e2m1[codes] * np.repeat(s, 16, axis=1) * g


@pytest.fixture(scope="module")
def tiny():
    w = synth.TINY
    gate, up = w.activations()
    aq, as_, ga = oracle.quantize(gate, up)
    wq, ws, gw = oracle.quantize(w.weight())
    return w, aq, as_, ga, wq, ws, gw


def test_tiny_gemm_matches_fp64_dequant_matmul(tiny):
    w, aq, as_, ga, wq, ws, gw = tiny
    d = oracle.gemm_rows(aq, as_, w.m, ga, wq, ws, w.n, gw, w.k, np.arange(w.m_pad))
    A = dequant(aq, as_, w.m, w.k, 1.0)
    W = dequant(wq, ws, w.n, w.k, 1.0)
    ref = (A @ W.T) * (float(ga) * float(gw))
    ok = boundary_distance(ref) > 1e-9
    assert ok.mean() > 0.999
    want = round_f64_to_bf16(ref)
    np.testing.assert_array_equal(d[ok], want[ok])
    assert np.abs(oracle.bf16_bits_to_f32(d)).max() > 0


def test_gemm_one_hot_weight_is_a_gather(tiny):
    """W rows with a single non-zero code: D[m, j] = RN(ga gw v(SA) v(SW) a w) exactly."""
    w, aq, as_, ga, _, _, _ = tiny
    rng = np.random.default_rng(3)
    n, k = 48, w.k
    cpad = oracle.scale_cols(k)
    wq = np.zeros((n, k // 2), dtype=np.uint8)
    ws = np.zeros(oracle.scale_bytes(n, k), dtype=np.uint8)
    pos = rng.integers(0, k, size=n)
    code = rng.integers(1, 16, size=n)
    sbyte = rng.integers(1, 127, size=n)
    for j in range(n):
        kk = int(pos[j])
        wq[j, kk // 2] = int(code[j]) << (4 * (kk & 1))
        ws[oracle.scale_offset(j, kk // 16, cpad)] = int(sbyte[j])
    gw = 0.037109375
    rows = np.arange(0, w.m, 7)
    d = oracle.gemm_rows(aq, as_, w.m, ga, wq, ws, n, gw, k, rows)
    for i, r in enumerate(rows):
        for j in range(n):
            kk = int(pos[j])
            ab = int(aq[r, kk // 2])
            ac = (ab >> 4) if kk & 1 else ab & 15
            sa = int(as_[oracle.scale_offset(int(r), kk // 16, cpad)])
            v = (Fraction(ga) * Fraction(gw) * exact.ue4m3_bits_value(sa) * exact.ue4m3_bits_value(int(sbyte[j]))
                 * exact.e2m1_bits_value(ac) * exact.e2m1_bits_value(int(code[j])))
            want = exact.rn_bf16_bits(v)
            assert d[i, j] == want, (r, j)


def test_gemm_all_ones_weight_is_a_row_sum(tiny):
    """W = all code 1.0 with scale 1.0 and gw = 1: D[m, :] = RN(ga * sum_k deq(A[m, k]))."""
    w, aq, as_, ga, _, _, _ = tiny
    n, k = 32, w.k
    wq = np.full((n, k // 2), 0x22, dtype=np.uint8)
    ws = np.zeros(oracle.scale_bytes(n, k), dtype=np.uint8)
    cpad = oracle.scale_cols(k)
    for j in range(n):
        for b in range(k // 16):
            ws[oracle.scale_offset(j, b, cpad)] = 0x38
    rows = np.arange(w.m)
    d = oracle.gemm_rows(aq, as_, w.m, ga, wq, ws, n, 1.0, k, rows)
    A = dequant(aq, as_, w.m, k, 1.0)  # multiples of 2^-10 below 2^12: row sums exact in fp64
    for r in rows:
        want = exact.rn_bf16_bits(Fraction(ga) * Fraction(float(A[r].sum())))
        assert (d[r] == want).all(), r


def test_gemm_operand_swap_is_a_transpose(tiny):
    w, aq, as_, ga, wq, ws, gw = tiny
    d = oracle.gemm_rows(aq, as_, w.m, ga, wq, ws, w.n, gw, w.k, np.arange(w.m))
    dt = oracle.gemm_rows(wq, ws, w.n, gw, aq, as_, w.m, ga, w.k, np.arange(w.n))
    np.testing.assert_array_equal(d, dt.T)


def test_gemm_padding_rows_are_positive_zero():
    w = synth.Workload("t", m=37, n=32, k=64, seed=2, swiglu=False)
    x, = w.activations()
    aq, as_, ga = oracle.quantize(x)
    wq, ws, gw = oracle.quantize(w.weight())
    d = oracle.gemm_rows(aq, as_, w.m, ga, wq, ws, w.n, gw, w.k, np.arange(w.m, w.m_pad))
    assert (d == 0).all()


def test_gemm_rejects_out_of_range_rows(tiny):
    w, aq, as_, ga, wq, ws, gw = tiny
    with pytest.raises(ValueError):
        oracle.gemm_rows(aq, as_, w.m, ga, wq, ws, w.n, gw, w.k, [w.m_pad])


def test_gemm_exact_ties_round_to_even():
    """Row sums placed exactly on bf16 rounding boundaries (ga = gw = 1, W = all 1.0):
    1 + 2^-8 -> 1 (even), 1 + 3*2^-8 -> 1 + 2^-6 (even), and their negatives."""
    k, n = 64, 16
    cpad = oracle.scale_cols(k)
    aq = np.zeros((16, k // 2), dtype=np.uint8)
    as_ = np.zeros(oracle.scale_bytes(16, k), dtype=np.uint8)
    # row 0: 1.0 (code 2, scale 1.0 = 0x38) + 0.5 * 2^-7 (code 1, scale 4 * 2^-9 = 0x04)
    # row 1: 1.0 + 1.5 * 2^-7 (code 3, scale 0x04)
    # rows 2, 3: the negatives (sign bit 8 on both codes)
    for r, (c0, c1) in enumerate([(2, 1), (2, 3), (10, 9), (10, 11)]):
        aq[r, 0] = c0
        aq[r, 8] = c1
        as_[oracle.scale_offset(r, 0, cpad)] = 0x38
        as_[oracle.scale_offset(r, 1, cpad)] = 0x04
    wq = np.full((n, k // 2), 0x22, dtype=np.uint8)
    ws = np.zeros(oracle.scale_bytes(n, k), dtype=np.uint8)
    for j in range(n):
        for b in range(k // 16):
            ws[oracle.scale_offset(j, b, cpad)] = 0x38
    d = oracle.gemm_rows(aq, as_, 16, 1.0, wq, ws, n, 1.0, k, [0, 1, 2, 3])
    assert (d[0] == 0x3F80).all()          # 1 + 2^-8 -> 1.0
    assert (d[1] == 0x3F82).all()          # 1 + 3 * 2^-8 -> 1 + 2^-6
    assert (d[2] == 0xBF80).all()
    assert (d[3] == 0xBF82).all()
