"""Pins for the oracle's quantizer: formats, global scale, block scale, E2M1 codes,
packing, padding and the spec invariants (steps O3-O8).

Formats: E2M1 data with vector-16 UE4M3 block scales and an FP32 global scale
("FC2 NVFP4 Scheduling Results", section "Canonical Operation"). Padding rows
are zero; the block-scale buffer is zero-initialised before packing
(component-2 NSYS summary, "block_scale_zero" keys).
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import exact


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def prev_f32(g: float) -> float:
    return float(np.nextafter(np.float32(g), np.float32(0)))


def next_f32(g: float) -> float:
    return float(np.nextafter(np.float32(g), np.float32(np.inf)))


# ---- formats ----------------------------------------------------------------------

def test_ue4m3_decode_matches_torch_float8_e4m3fn():
    lib = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(127):
        assert oracle.ue4m3_value(b) == lib[b], b
        assert Fraction(oracle.ue4m3_value(b)) == exact.ue4m3_bits_value(b)
    assert oracle.ue4m3_value(0x7E) == 448.0
    vals = [oracle.ue4m3_value(b) for b in range(127)]
    assert all(a < b for a, b in zip(vals, vals[1:]))  # strictly increasing in the byte


def test_e2m1_decode_matches_bit_fields():
    for c in range(16):
        assert Fraction(oracle.e2m1_value(c)) == exact.e2m1_bits_value(c)
    assert sorted({abs(oracle.e2m1_value(c)) for c in range(16)}) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


# ---- O4 global scale ---------------------------------------------------------------

def test_global_scale_exhaustive_over_bf16_amax():
    """For every positive finite bf16 amax: 2688 g >= amax and 2688 prev(g) < amax."""
    for bits in range(1, 0x7F80):
        amax = exact.bf16_value(bits)
        g = oracle.global_scale(float(amax))
        assert g == f32(g) and g > 0
        assert Fraction(g) * 2688 >= amax, hex(bits)
        p = prev_f32(g)
        assert p == 0 or Fraction(p) * 2688 < amax, hex(bits)
    assert oracle.global_scale(0.0) == 0.0
    assert oracle.global_scale(2688.0) == 1.0
    assert oracle.global_scale(448.0 * 6 * 2.0 ** -20) == 2.0 ** -20


# ---- O5 block scale ----------------------------------------------------------------

def brute_block_scale(bmax: Fraction, g: Fraction) -> int:
    for e in range(127):
        if exact.ue4m3_bits_value(e) * 6 * g >= bmax:
            return e
    raise AssertionError("no scale")


def test_block_scale_brute_force_random():
    rng = np.random.default_rng(5)
    for _ in range(4000):
        amax_bits = int(rng.integers(0x3000, 0x4800))
        amax = exact.bf16_value(amax_bits)
        g = oracle.global_scale(float(amax))
        # block max: a bf16 value at most amax
        bm_bits = int(rng.integers(0, amax_bits + 1))
        bmax = exact.bf16_value(bm_bits)
        want = brute_block_scale(bmax, Fraction(g))
        assert oracle.block_scale(float(bmax), g) == want, (hex(amax_bits), hex(bm_bits))
    # the amax block takes the largest scale byte
    for amax_bits in [0x3F80, 0x4120, 0x42F6, 0x3C23, 0x0001, 0x7F7F]:
        amax = float(exact.bf16_value(amax_bits))
        g = oracle.global_scale(amax)
        assert oracle.block_scale(amax, g) == 0x7E
    assert oracle.block_scale(0.0, 0.5) == 0
    assert oracle.block_scale(0.0, 0.0) == 0


# ---- O6 E2M1 codes -------------------------------------------------------------------

def brute_code(y: Fraction, neg: bool, s: int, g: Fraction) -> int:
    sign = 8 if neg else 0
    if s == 0:
        return sign
    t = abs(y) / (exact.ue4m3_bits_value(s) * g)
    best = None
    for idx, v in enumerate(exact.E2M1_GRID):
        d = abs(t - v)
        if best is None or d < best[0] or (d == best[0] and idx % 2 == 0):
            best = (d, idx)
    return sign | best[1]


def test_e2m1_code_brute_force_random():
    rng = np.random.default_rng(11)
    for _ in range(20000):
        g = f32(float(rng.uniform(1e-4, 1.0)))
        s = int(rng.integers(1, 127))
        unit = exact.ue4m3_bits_value(s) * Fraction(g)
        t = Fraction(float(rng.uniform(0, 6.0)))
        ybits = exact.rn_bf16_bits(t * unit)
        if rng.random() < 0.5:
            ybits |= 0x8000
        y = exact.bf16_value(ybits)
        want = brute_code(y, bool(ybits & 0x8000), s, Fraction(g))
        assert oracle.e2m1_code(float(y) if y != 0 else (-0.0 if ybits & 0x8000 else 0.0), s, g) == want


def test_e2m1_code_ties_go_to_even():
    """Hand-built ties: y exactly on each of the seven midpoints, for power-of-two g and
    scales whose unit keeps y representable in bf16."""
    mids = [Fraction(1, 4), Fraction(3, 4), Fraction(5, 4), Fraction(7, 4), Fraction(5, 2),
            Fraction(7, 2), Fraction(5)]
    # expected magnitude index at each midpoint: the even one of its two neighbours
    want_idx = [0, 2, 2, 4, 4, 6, 6]
    for g in [1.0, 2.0 ** -10, 0.5]:
        for s in [0x38, 0x30, 0x40, 0x39, 0x01, 0x04]:  # 1, 0.5, 2, 1.125, 2^-9, 2^-7
            unit = exact.ue4m3_bits_value(s) * Fraction(g)
            for mid, idx in zip(mids, want_idx):
                y = mid * unit
                yb = exact.rn_bf16_bits(y)
                if exact.bf16_value(yb) != y:
                    continue  # not representable in bf16: not a tie case
                assert oracle.e2m1_code(float(y), s, g) == idx, (g, hex(s), mid)
                assert oracle.e2m1_code(-float(y), s, g) == 8 | idx
                # just above / below the midpoint
                up = exact.bf16_value(yb + 1)
                dn = exact.bf16_value(yb - 1)
                assert oracle.e2m1_code(float(up), s, g) == brute_code(up, False, s, Fraction(g))
                assert oracle.e2m1_code(float(dn), s, g) == brute_code(dn, False, s, Fraction(g))
    # signed zero keeps its sign; zero scale gives magnitude 0
    assert oracle.e2m1_code(-0.0, 0x38, 1.0) == 0x8
    assert oracle.e2m1_code(0.0, 0x38, 1.0) == 0x0
    assert oracle.e2m1_code(-3.0, 0, 1.0) == 0x8
    # subnormal y rounds to a signed zero code
    assert oracle.e2m1_code(-float(exact.bf16_value(0x0001)), 0x38, 1.0) == 0x8


# ---- O7/O8 whole tensors ---------------------------------------------------------------

def unpack_codes(qdata: np.ndarray) -> np.ndarray:
    """Independent unpacker: element 2j is the low nibble of byte j, 2j+1 the high."""
    lo = qdata & 0x0F
    hi = qdata >> 4
    out = np.empty((qdata.shape[0], qdata.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


@pytest.fixture(scope="module")
def tiny_quant():
    w = synth.TINY
    gate, up = w.activations()
    qd, sc, g, y = oracle.quantize(gate, up, return_y=True)
    return w, gate, up, qd, sc, g, y


def test_tiny_y_matches_library_swiglu(tiny_quant):
    w, gate, up, qd, sc, g, y = tiny_quant
    tab = oracle.silu_table()
    s = torch.from_numpy(tab[gate].astype(np.int16)).view(torch.bfloat16)
    u = torch.from_numpy(up.astype(np.int16)).view(torch.bfloat16)
    want = (s * u).view(torch.int16).numpy().astype(np.uint16)
    np.testing.assert_array_equal(y, want)


def test_tiny_quantization_brute_force(tiny_quant):
    """Every block scale and code of the tiny config against exact rationals."""
    w, gate, up, qd, sc, g, y = tiny_quant
    k = w.k
    yf = oracle.bf16_bits_to_f32(y).astype(np.float64)
    amax = np.abs(yf).max()
    assert g == oracle.global_scale(float(amax))
    G = Fraction(g)
    codes = unpack_codes(qd)
    cpad = oracle.scale_cols(k)
    n_sub = 0
    for r in range(w.m):
        for b in range(k // 16):
            blk = y[r, b * 16:(b + 1) * 16]
            vals = [exact.bf16_value(int(v)) for v in blk]
            bmax = max(abs(v) for v in vals)
            s = brute_block_scale(bmax, G)
            assert sc[oracle.scale_offset(r, b, cpad)] == s
            n_sub += (1 <= s <= 7)
            if r % 16 == 0:  # codes: exact check on every 16th row (the scale check covers all)
                for t in range(16):
                    want = brute_code(vals[t], bool(int(blk[t]) & 0x8000), s, G)
                    assert codes[r, b * 16 + t] == want
    assert n_sub == 0  # no subnormal block scale on the tiny config


def test_tiny_invariants(tiny_quant):
    """Spec invariants: (1) v(S) * 6 * g >= block absmax for every block;
    (2) every scale byte is a UE4M3 value (<= 0x7E, no sign) and every code decodes into
    the E2M1 set; (3) re-quantizing the dequantized tensor returns the same bytes."""
    w, gate, up, qd, sc, g, y = tiny_quant
    k = w.k
    cpad = oracle.scale_cols(k)
    G = Fraction(g)
    codes = unpack_codes(qd)
    yf = oracle.bf16_bits_to_f32(y).astype(np.float64)
    # (1)
    for r in range(w.m):
        for b in range(k // 16):
            s = int(sc[oracle.scale_offset(r, b, cpad)])
            bmax = Fraction(float(np.abs(yf[r, b * 16:(b + 1) * 16]).max()))
            assert exact.ue4m3_bits_value(s) * 6 * G >= bmax
    # (2)
    assert sc.max() <= 0x7E
    assert set(np.unique(codes).tolist()) <= set(range(16))
    # (3) dequantize exactly, then requantize with the oracle's own steps
    deq = np.zeros((w.m, k), dtype=np.float64)
    for r in range(w.m):
        for b in range(k // 16):
            s = int(sc[oracle.scale_offset(r, b, cpad)])
            v = oracle.ue4m3_value(s) * g
            for t in range(16):
                deq[r, b * 16 + t] = oracle.e2m1_value(int(codes[r, b * 16 + t])) * v  # exact
    amax2 = float(np.abs(deq).max())
    g2 = oracle.global_scale(amax2)
    assert g2 == g
    for r in range(0, w.m, 3):
        for b in range(k // 16):
            blk = deq[r, b * 16:(b + 1) * 16]
            s2 = oracle.block_scale(float(np.abs(blk).max()), g2)
            assert s2 == sc[oracle.scale_offset(r, b, cpad)]
            for t in range(16):
                assert oracle.e2m1_code(float(blk[t]), s2, g2) == codes[r, b * 16 + t]


def test_padding_rows_and_scale_padding_are_zero():
    """A ragged M: rows [m, m_pad) of QDATA are zero and every scale byte outside
    the real (row < m_pad, column < k/16) region is zero."""
    m, k = 37, 96  # m_pad = 48, scale rows 128, scale cols roundup(6,4) = 8
    x = synth.normal_bf16(m, k, seed=3, tag=9, sigma=1.0)
    qd, sc, g = oracle.quantize(x)
    assert qd.shape == (48, 48)
    assert (qd[m:] == 0).all()
    cpad = oracle.scale_cols(k)
    assert cpad == 8 and sc.size == 128 * 8
    covered = np.zeros(sc.size, dtype=bool)
    for r in range(48):
        for c in range(k // 16):
            covered[oracle.scale_offset(r, c, cpad)] = True
    assert (sc[~covered] == 0).all()
    for r in range(m, 48):
        for c in range(k // 16):
            assert sc[oracle.scale_offset(r, c, cpad)] == 0


def test_zero_tensor_quantizes_to_zero():
    x = np.zeros((16, 64), dtype=np.uint16)
    x[3, 5] = 0x8000  # -0 keeps its sign code
    qd, sc, g = oracle.quantize(x)
    assert g == 0.0
    assert (sc == 0).all()
    codes = unpack_codes(qd)
    assert codes[3, 5] == 8
    codes[3, 5] = 0
    assert (codes == 0).all()


def test_plain_quantize_is_y_equals_x():
    x = synth.normal_bf16(32, 128, seed=4, tag=4, sigma=1.0)
    _, _, _, y = oracle.quantize(x, return_y=True)
    np.testing.assert_array_equal(y, x)


def test_amax_is_a_magnitude():
    """The tensor absmax uses |y|: a tensor whose largest magnitude is negative."""
    x = np.zeros((16, 32), dtype=np.uint16)
    x[0, 0] = 0x3F80   # +1
    x[5, 7] = 0xC120   # -10
    qd, sc, g = oracle.quantize(x)
    assert g == oracle.global_scale(10.0)
    assert Fraction(g) * 2688 >= 10
