"""Pins for the oracle's modulated quantization (step O13).

The pages list a fused modulation next to the NVFP4 boundaries of the QKV and FC1
inputs (the component-2 summary's residual components: "modulation" launches;
the FC2 production profile's configuration flags the modulate fusion) without a
formula. O13 reads it as adaLN modulation, y = x (1 + scale[k]) + shift[k], in the
kernel's precision: m = RN_fp32(1 + scale), one fused multiply-add rounded to
fp32, then one rounding to bf16. These tests rebuild that value from exact
fractions and an exact fp32 rounding written here, on random and edge triples,
and check that the quantized bytes are those of O3-O8 applied to it.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact


def rn_f32_exact(v: Fraction) -> Fraction:
    """Round an exact value to the nearest fp32 (ties to even), as a Fraction."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = max(exact.floor_log2(a), -126)
    q = Fraction(2) ** (e - 23)
    n = exact.round_half_even(a / q)
    r = n * q
    assert r < Fraction(2) ** 128
    return r if v > 0 else -r


def modulate_exact(x: int, s: int, b: int) -> int:
    xv, sv, bv = exact.bf16_value(x), exact.bf16_value(s), exact.bf16_value(b)
    m = Fraction(float(np.float32(1.0) + np.float32(float(sv))))  # IEEE single add
    y32 = rn_f32_exact(xv * m + bv)
    return exact.rn_bf16_bits(y32)


def finite_bf16(rng, n, lo_exp=-20, hi_exp=20):
    sign = rng.integers(0, 2, n) << 15
    e = rng.integers(127 + lo_exp, 127 + hi_exp, n) << 7
    f = rng.integers(0, 128, n)
    return (sign | e | f).astype(np.uint16)


def test_random_triples_match_exact():
    rng = np.random.default_rng(13)
    n = 6000
    xs, ss, bs = finite_bf16(rng, n), finite_bf16(rng, n, -30, 2), finite_bf16(rng, n)
    for x, s, b in zip(xs, ss, bs):
        got = oracle.modulate_bf16(int(x), int(s), int(b))
        want = modulate_exact(int(x), int(s), int(b))
        if want == 0:
            assert got & 0x7FFF == 0
        else:
            assert got == want, (hex(x), hex(s), hex(b), hex(got), hex(want))


@pytest.mark.parametrize("x,s,b", [
    (0x4040, 0xBF80, 0x3F80),   # scale -1: m = 0, y = shift
    (0x3F80, 0x3380, 0x0000),   # scale 2^-24: 1 + s rounds to 1 in fp32
    (0x3F81, 0x3400, 0x0000),   # scale 2^-23: exact in fp32
    (0x3F80, 0x3F80, 0xC000),   # 1 * 2 - 2 = 0
    (0x0001, 0x3F80, 0x0000),   # smallest subnormal x, doubled
    (0x7F7F, 0x3F00, 0x0000),   # largest finite x times 1.5 -> overflows bf16 rounding
    (0x3F80, 0x0000, 0x3B80),   # 1 + 2^-8: an exact bf16 tie
    (0x3F80, 0x0000, 0x3B81),   # just above the tie
    (0xBF80, 0x0000, 0xBB80),   # negative tie
])
def test_edge_triples(x, s, b):
    got = oracle.modulate_bf16(x, s, b)
    xv = exact.bf16_value(x) * Fraction(float(np.float32(1.0) + np.float32(float(exact.bf16_value(s)))))
    v = rn_f32_exact(xv + exact.bf16_value(b)) if abs(xv + exact.bf16_value(b)) < Fraction(2) ** 128 else None
    if v is None or abs(v) >= Fraction(2) ** 128:
        assert got & 0x7FFF == 0x7F80
    elif v == 0:
        assert got == 0x0000
    else:
        assert got == exact.rn_bf16_bits(v), (hex(got), hex(exact.rn_bf16_bits(v)))


def test_tie_rounds_to_even():
    assert oracle.modulate_bf16(0x3F80, 0x0000, 0x3B80) == 0x3F80   # 1 + 2^-8 -> 1 (even)
    assert oracle.modulate_bf16(0x3F81, 0x0000, 0x3B80) == 0x3F82   # (1 + 2^-7) + 2^-8 -> up to even


def test_quantize_modulate_is_quantize_of_modulated():
    m, k = 40, 192
    x = synth.normal_bf16(m, k, seed=41, tag=1, sigma=1.0)
    sc = synth.normal_bf16(1, k, seed=41, tag=2, sigma=0.3)[0]
    sh = synth.normal_bf16(1, k, seed=41, tag=3, sigma=0.1)[0]
    qd, scl, g, y = oracle.quantize_modulate(x, sc, sh, return_y=True)
    want_y = np.array([[modulate_exact(int(x[r, c]), int(sc[c]), int(sh[c])) for c in range(k)] for r in range(m)],
                      dtype=np.uint16)
    nz = want_y != 0
    assert (y[nz] == want_y[nz]).all() and ((y[~nz] & 0x7FFF) == 0).all()
    rq, rs, rg = oracle.quantize(y)
    assert (qd == rq).all() and (scl == rs).all() and g == rg
