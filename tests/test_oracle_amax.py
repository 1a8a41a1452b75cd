"""Pins for the oracle's single-read producer (O11): quantization with an amax the
caller supplies instead of the tensor maximum.

The pages derive the global scale from the data's own amax ("FC2 NVFP4 Scheduling
Results", "Canonical Operation"; the component-2 summary's nvfp4 conclusion names
that dependency as the one an exact fused producer must synchronize on). O11 takes
amax as an input; these tests pin it by brute force in exact rational arithmetic on
small tensors, by a scaling law of the format, and by closed forms for amax = 0.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact

E2M1 = [Fraction(v) for v in ("0", "0.5", "1", "1.5", "2", "3", "4", "6")]


def global_scale_exact(amax: Fraction) -> Fraction:
    """Smallest fp32 g with 2688 g >= amax, by walking fp32 bit patterns."""
    if amax <= 0:
        return Fraction(0)
    bits = exact.f32_bits(float(amax / 2688))
    while exact.f32_value(exact.bits_f32(bits)) * 2688 < amax:
        bits += 1
    while bits > 1 and exact.f32_value(exact.bits_f32(bits - 1)) * 2688 >= amax:
        bits -= 1
    return exact.f32_value(exact.bits_f32(bits))


def brute_block(vals, g: Fraction):
    """(scale byte, codes) of one 16-element block by exhaustive search: the smallest
    UE4M3 byte whose range covers the block maximum (126 if none does), then the
    nearest E2M1 magnitude of |y| / unit, ties to the even code, saturating at 6."""
    bmax = max(abs(v) for v in vals)
    s = 126
    for e in range(127):
        if exact.ue4m3_bits_value(e) * 6 * g >= bmax:
            s = e
            break
    unit = exact.ue4m3_bits_value(s) * g
    codes = []
    for v in vals:
        a = abs(v)
        if s == 0 or unit == 0:
            idx = 0 if (s == 0 or a == 0) else 7
        else:
            q = a / unit
            best = None
            for i, mag in enumerate(E2M1):
                d = abs(q - mag)
                if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
                    best = (d, i)
            idx = best[1]
        codes.append(idx)
    return s, codes


def oracle_codes(qd: np.ndarray, m: int, k: int) -> np.ndarray:
    lo = qd[:m] & 15
    hi = qd[:m] >> 4
    out = np.empty((m, k), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def check_brute(x, up, amax_value: float, m: int, k: int):
    qd, sc, g = oracle.quantize_amax(x, up, amax_value)
    _, _, _, y = oracle.quantize(x, up, return_y=True)
    gx = global_scale_exact(Fraction(amax_value) if amax_value == amax_value else Fraction(0))
    assert Fraction(g) == gx, (g, gx)
    codes = oracle_codes(qd, m, k)
    cpad = oracle.scale_cols(k)
    for r in range(m):
        for b in range(k // 16):
            ys = [int(t) for t in y[r, b * 16:(b + 1) * 16]]
            vals = [exact.bf16_value(t) for t in ys]
            s, mags = brute_block(vals, gx)
            assert sc[oracle.scale_offset(r, b, cpad)] == s, (r, b)
            for t in range(16):
                want = mags[t] | (8 if ys[t] & 0x8000 else 0)
                assert codes[r, b * 16 + t] == want, (r, b, t)
    return qd, sc, g


def small_inputs(m=24, k=64, seed=3):
    gate = synth.normal_bf16(m, k, seed=seed, tag=1, sigma=1.0)
    up = synth.normal_bf16(m, k, seed=seed, tag=2, sigma=1.0)
    return gate, up


def true_amax(x, up) -> float:
    _, _, _, y = oracle.quantize(x, up, return_y=True)
    return float(np.abs(oracle.bf16_bits_to_f32(y).astype(np.float64)).max())


@pytest.mark.parametrize("factor", [1.0, 1.5, 7.0, 0.25, 1e-3])
def test_given_amax_brute_force(factor):
    """Every scale byte and code equals the exhaustive-search result, for amax at,
    above and below the true maximum (below: the saturating blocks)."""
    gate, up = small_inputs()
    check_brute(gate, up, true_amax(gate, up) * factor, 24, 64)


def test_given_true_amax_equals_two_pass():
    gate, up = small_inputs(m=40, k=128, seed=9)
    a = oracle.quantize(gate, up)
    b = oracle.quantize_amax(gate, up, true_amax(gate, up))
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all() and a[2] == b[2]


def test_doubling_amax_shifts_normal_scales_by_one_binade():
    """g(2 amax) = 2 g(amax) exactly, so a block whose scale byte S is at least 16
    (v(S) normal, and so is v(S - 8) = v(S) / 2) gets S - 8 and keeps every code."""
    gate, up = small_inputs(m=48, k=256, seed=5)
    am = true_amax(gate, up)
    q1, s1, g1 = oracle.quantize_amax(gate, up, am)
    q2, s2, g2 = oracle.quantize_amax(gate, up, 2 * am)
    assert g2 == 2 * g1
    cpad = oracle.scale_cols(256)
    checked = 0
    for r in range(48):
        for b in range(16):
            o = oracle.scale_offset(r, b, cpad)
            if s1[o] >= 16:
                assert s2[o] == s1[o] - 8
                assert (q1[r, b * 8:(b + 1) * 8] == q2[r, b * 8:(b + 1) * 8]).all()
                checked += 1
    assert checked > 700


@pytest.mark.parametrize("amax", [0.0, -1.0, float("nan")])
def test_zero_negative_or_nan_amax(amax):
    """g = 0: every block with a nonzero element saturates (byte 126, codes +-6 on
    nonzero elements, signed zero elsewhere); all-zero blocks keep byte 0."""
    x = synth.normal_bf16(16, 64, seed=2, tag=1, sigma=1.0)
    x[3, :16] = 0
    x[5, 16:32] = 0x8000
    qd, sc, g = oracle.quantize_amax(x, None, amax)
    assert g == 0.0
    codes = oracle_codes(qd, 16, 64)
    cpad = oracle.scale_cols(64)
    for r in range(16):
        for b in range(4):
            blk = x[r, b * 16:(b + 1) * 16]
            nz = (blk & 0x7FFF) != 0
            assert sc[oracle.scale_offset(r, b, cpad)] == (126 if nz.any() else 0)
            want = np.where(nz, 7, 0) | np.where(blk & 0x8000, 8, 0)
            assert (codes[r, b * 16:(b + 1) * 16] == want).all()


def test_plain_given_amax_brute_force():
    x = synth.normal_bf16(20, 128, seed=4, tag=7, sigma=3.0)
    check_brute(x, None, float(np.abs(oracle.bf16_bits_to_f32(x)).max()) * 3.25, 20, 128)
