"""Pins for the oracle's silu and SwiGLU product (steps O1-O2).

The component-2 NSYS summary (keys "swiglu_silu_total_ms" and
"swiglu_multiply_total_ms") shows the activation as a bf16 silu followed by a
bf16 multiply; the oracle reads silu as correctly rounded to bf16 and the
product as one rounding of the exact bf16 x bf16 product.
"""
import decimal
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

CTX = decimal.Context(prec=60, Emax=decimal.MAX_EMAX, Emin=decimal.MIN_EMIN)


def silu_decimal(x: Fraction) -> Fraction:
    """x / (1 + e^-x) to about 55 significant digits."""
    d = CTX.divide(decimal.Decimal(x.numerator), decimal.Decimal(x.denominator))
    e = CTX.exp(CTX.minus(d))
    s = CTX.divide(d, CTX.add(decimal.Decimal(1), e))
    return Fraction(s)


def expected_silu_bits(bits: int):
    """Correctly rounded silu of a finite bf16 and the relative distance of the
    high-precision value to the nearest bf16 rounding boundary."""
    x = exact.bf16_value(bits)
    neg = bool(bits & 0x8000)
    if x == 0:
        return bits, None
    if x > 1000:  # e^-x < 1e-434: silu(x) = x (1 - tiny), rounds to x
        return bits, None
    if x < -1000:  # |silu(x)| < 1000 e^-1000, far below the smallest bf16 subnormal
        return 0x8000, None
    s = silu_decimal(x)
    b = exact.rn_bf16_bits(s, negative_zero=neg)
    # distance to the rounding boundaries around s (midpoints of neighbouring bf16s)
    a = abs(s)
    e = max(exact.floor_log2(a), -126) if a != 0 else -126
    q = Fraction(2) ** (e - 7)
    frac_part = (a / q) - (a / q).numerator // (a / q).denominator
    dist = abs(frac_part - Fraction(1, 2)) * q / a if a != 0 else None
    return b, dist


@pytest.fixture(scope="module")
def silu_tab():
    return oracle.silu_table()


def test_silu_exhaustive_against_decimal(silu_tab):
    """All 65,280 finite bf16 inputs: the oracle's silu is the correctly rounded value."""
    mism = []
    min_dist = Fraction(1)
    for bits in range(65536):
        if (bits & 0x7F80) == 0x7F80:
            continue
        want, dist = expected_silu_bits(bits)
        if dist is not None and dist < min_dist:
            min_dist = dist
        if int(silu_tab[bits]) != want:
            mism.append((hex(bits), hex(int(silu_tab[bits])), hex(want)))
    assert not mism, f"{len(mism)} mismatches, first {mism[:5]}"
    # The 60-digit evaluation is far from every rounding boundary, so the
    # decimal reference itself is unambiguous.
    assert min_dist > Fraction(1, 10 ** 50)


def test_silu_special_cases():
    assert oracle.silu_bf16(0x0000) == 0x0000          # silu(+0) = +0
    assert oracle.silu_bf16(0x8000) == 0x8000          # silu(-0) = -0
    assert oracle.silu_bf16(0x42C8) == 0x42C8          # silu(100) rounds to 100
    assert oracle.silu_bf16(0xC2C8) == 0x8000          # silu(-100) = -100 e^-100 underflows to -0
    assert oracle.silu_bf16(0x7F7F) == 0x7F7F          # largest finite: x
    assert oracle.silu_bf16(0xFF7F) == 0x8000
    # silu(1) = 0.7310585786... -> bf16 0.73046875 (0x3F3B)
    assert oracle.silu_bf16(0x3F80) == 0x3F3B
    # silu(-1) = -0.2689414213... -> bf16 -0.26953125 (0xBE8A)
    assert oracle.silu_bf16(0xBF80) == 0xBE8A


def test_silu_table_matches_scalar(silu_tab):
    for bits in [0, 1, 0x3F80, 0xBF80, 0x4000, 0xC0A0, 0x0080, 0x8080, 0x7F7F]:
        assert int(silu_tab[bits]) == oracle.silu_bf16(bits)


def test_swiglu_product_matches_torch_bf16_multiply(silu_tab):
    """O2 against a library routine: torch's CPU bf16 multiply (float product, one
    round to bf16) on random normal-range operands, where the float product is exact."""
    rng = np.random.default_rng(1234)
    gate = (rng.standard_normal(20000).astype(np.float32) * 3)
    up = (rng.standard_normal(20000).astype(np.float32) * 3)
    gb = torch.from_numpy(gate).to(torch.bfloat16)
    ub = torch.from_numpy(up).to(torch.bfloat16)
    gbits = gb.view(torch.int16).numpy().astype(np.uint16)
    ubits = ub.view(torch.int16).numpy().astype(np.uint16)
    s = torch.from_numpy(silu_tab[gbits].astype(np.int16)).view(torch.bfloat16)
    want = (s * ub).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([oracle.swiglu_bf16(int(a), int(b)) for a, b in zip(gbits, ubits)], dtype=np.uint16)
    prod = s.float() * ub.float()
    normal = (prod.abs() >= 2.0 ** -126).numpy() | (prod == 0).numpy()
    assert normal.mean() > 0.99
    np.testing.assert_array_equal(got[normal], want[normal])


def test_swiglu_exact_rounding_small_products():
    """One rounding of the exact product, also where the product is below the
    smallest normal (torch's float product would round twice there)."""
    rng = np.random.default_rng(7)
    for _ in range(3000):
        g = int(rng.integers(0, 65536))
        u = int(rng.integers(0, 65536))
        if (g & 0x7F80) == 0x7F80 or (u & 0x7F80) == 0x7F80:
            continue
        s = oracle.silu_bf16(g)
        p = exact.bf16_value(s) * exact.bf16_value(u)
        neg = bool((s ^ u) & 0x8000)
        want = exact.rn_bf16_bits(p, negative_zero=neg)
        if (want & 0x7F80) == 0x7F80:
            continue  # overflow is outside the method's domain
        assert oracle.swiglu_bf16(g, u) == want, (hex(g), hex(u))
    # hand-built: tiny operands whose exact product is a bf16 subnormal
    for s_bits, u_bits in [(0x0001, 0x3F80), (0x00FF, 0x3F01), (0x0100, 0x3E80)]:
        g = s_bits
        s = oracle.silu_bf16(g)
        p = exact.bf16_value(s) * exact.bf16_value(u_bits)
        assert oracle.swiglu_bf16(g, u_bits) == exact.rn_bf16_bits(p, negative_zero=bool((s ^ u_bits) & 0x8000))
