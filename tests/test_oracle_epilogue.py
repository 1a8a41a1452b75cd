"""Pins for the oracle's GEMM epilogue fusions (step O12).

The FC2 kernel's name on the pages carries a bf16 bias, and the step profile keeps
a gate/residual add after the GEMM (the FC2 production profile's components,
"remaining_gate_add"). O12 computes D1 = RN_bf16(X + bias[n]) with X the exact
block-scaled sum, then D = RN_bf16(res + gate[n] * D1). These tests rebuild X in
Python integers from the bit-level formats and round with the independent
fractions helpers, on cases chosen to hit exact cancellation, ties, sticky
alignment and subnormal results.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact

E2M1_2X = [0, 1, 2, 3, 4, 6, 8, 12]


def codes_of(qdata: np.ndarray, rows: int, k: int) -> np.ndarray:
    out = np.empty((rows, k), dtype=np.int64)
    lo = (qdata[:rows] & 15).astype(np.int64)
    hi = (qdata[:rows] >> 4).astype(np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def twice_e2m1(c: int) -> int:
    v = E2M1_2X[c & 7]
    return -v if c & 8 else v


def exact_sums(aq, as_, a_rows, ga, wq, ws, n, gw, k):
    """X[r, j] as Fractions for every activation row r < a_rows and column j < n."""
    ca = codes_of(aq, a_rows, k)
    cw = codes_of(wq, n, k)
    cpad = oracle.scale_cols(k)
    nb = k // 16
    A = np.vectorize(twice_e2m1)(ca)
    W = np.vectorize(twice_e2m1)(cw)
    SA = [[exact.ue4m3_bits_value(int(as_[oracle.scale_offset(r, b, cpad)])) for b in range(nb)]
          for r in range(a_rows)]
    SW = [[exact.ue4m3_bits_value(int(ws[oracle.scale_offset(j, b, cpad)])) for b in range(nb)]
          for j in range(n)]
    G = Fraction(ga) * Fraction(gw) / 4
    X = {}
    for r in range(a_rows):
        for j in range(n):
            tot = Fraction(0)
            for b in range(nb):
                dot = int(np.dot(A[r, b * 16:(b + 1) * 16], W[j, b * 16:(b + 1) * 16]))
                if dot:
                    tot += dot * SA[r][b] * SW[j][b]
            X[r, j] = G * tot
    return X


@pytest.fixture(scope="module")
def small():
    m, n, k = 12, 40, 64
    x = synth.normal_bf16(m, k, seed=31, tag=1, sigma=1.0)
    w = synth.normal_bf16(n, k, seed=31, tag=2, sigma=0.02)
    aq, as_, ga = oracle.quantize(x)
    wq, ws, gw = oracle.quantize(w)
    X = exact_sums(aq, as_, oracle.padded_rows(m), ga, wq, ws, n, gw, k)
    return dict(m=m, n=n, k=k, aq=aq, as_=as_, ga=ga, wq=wq, ws=ws, gw=gw, X=X)


def bias_patterns(X, m, n):
    """One bias per column: zero, cancellation of row 0's rounded value, near-ties,
    tiny (sticky only), huge (X only sticky), subnormal, negative zero."""
    out = np.zeros(n, dtype=np.uint16)
    for j in range(n):
        x0 = X[0, j]
        kind = j % 8
        if kind == 0:
            b = 0
        elif kind == 1:
            b = exact.rn_bf16_bits(-x0)
        elif kind == 2:
            b = exact.rn_bf16_bits(x0 * 3)
        elif kind == 3:
            b = 0x0001  # smallest subnormal
        elif kind == 4:
            b = 0x5F80  # 2^64
        elif kind == 5:
            b = 0x8000
        elif kind == 6:
            b = exact.rn_bf16_bits(-x0 * Fraction(255, 256))
        else:
            b = exact.rn_bf16_bits(Fraction(j - 20, 7))
        out[j] = b
    return out


def test_bias_only_matches_exact(small):
    s = small
    rows = list(range(oracle.padded_rows(s["m"])))
    bias = bias_patterns(s["X"], s["m"], s["n"])
    d1, d = oracle.gemm_rows_ex(s["aq"], s["as_"], s["m"], s["ga"], s["wq"], s["ws"], s["n"], s["gw"], s["k"], rows,
                                bias=bias)
    assert (d1 == d).all()
    for i, r in enumerate(rows):
        for j in range(s["n"]):
            want = exact.rn_bf16_bits(s["X"][r, j] + exact.bf16_value(int(bias[j])))
            assert d1[i, j] == want, (r, j, hex(d1[i, j]), hex(want))


def test_no_bias_equals_plain_gemm(small):
    s = small
    rows = [0, 3, 11, 15]
    plain = oracle.gemm_rows(s["aq"], s["as_"], s["m"], s["ga"], s["wq"], s["ws"], s["n"], s["gw"], s["k"], rows)
    d1, d = oracle.gemm_rows_ex(s["aq"], s["as_"], s["m"], s["ga"], s["wq"], s["ws"], s["n"], s["gw"], s["k"], rows,
                                bias=np.zeros(s["n"], dtype=np.uint16))
    assert (d1 == plain).all() and (d == plain).all()


def test_gated_residual_matches_exact(small):
    s = small
    m_pad = oracle.padded_rows(s["m"])
    rows = list(range(m_pad))
    bias = bias_patterns(s["X"], s["m"], s["n"])
    gate = synth.normal_bf16(1, s["n"], seed=32, tag=3, sigma=0.5)[0]
    gate[5] = 0x0000
    gate[6] = 0xBF80  # -1
    res = synth.normal_bf16(m_pad, s["n"], seed=32, tag=4, sigma=0.05)
    d1, d = oracle.gemm_rows_ex(s["aq"], s["as_"], s["m"], s["ga"], s["wq"], s["ws"], s["n"], s["gw"], s["k"], rows,
                                bias=bias, gate=gate, res=res)
    for i, r in enumerate(rows):
        for j in range(s["n"]):
            d1w = exact.rn_bf16_bits(s["X"][r, j] + exact.bf16_value(int(bias[j])))
            assert d1[i, j] == d1w
            v = exact.bf16_value(int(res[r, j])) + exact.bf16_value(int(gate[j])) * exact.bf16_value(d1w)
            want = exact.rn_bf16_bits(v)
            assert d[i, j] == want, (r, j, hex(d[i, j]), hex(want))


def test_residual_cancellation_gives_plus_zero(small):
    """res = -gate * D1 exactly: the sum is an exact zero and rounds to +0."""
    s = small
    rows = list(range(4))
    d1, _ = oracle.gemm_rows_ex(s["aq"], s["as_"], s["m"], s["ga"], s["wq"], s["ws"], s["n"], s["gw"], s["k"], rows,
                                bias=np.zeros(s["n"], dtype=np.uint16))
    res = np.zeros((oracle.padded_rows(s["m"]), s["n"]), dtype=np.uint16)
    res[:4] = d1 ^ 0x8000  # -D1 with gate = 1
    _, d = oracle.gemm_rows_ex(s["aq"], s["as_"], s["m"], s["ga"], s["wq"], s["ws"], s["n"], s["gw"], s["k"], rows,
                               res=res)
    assert (d == 0).all()


def test_gate_without_residual_rejected(small):
    s = small
    with pytest.raises(ValueError):
        oracle.gemm_rows_ex(s["aq"], s["as_"], s["m"], s["ga"], s["wq"], s["ws"], s["n"], s["gw"], s["k"], [0],
                            gate=np.zeros(s["n"], dtype=np.uint16))


def test_exact_tie_decided_by_tiny_bias():
    """X = 257/256 lies exactly halfway between the bf16 values 1 and 1 + 2^-7. With no
    bias it rounds to even (1.0); the smallest subnormal bias of either sign, or any
    tiny bias, must decide the side - the sticky bit of the aligned sum."""
    n, k = 16, 64
    cpad = oracle.scale_cols(k)
    aq = np.zeros((16, k // 2), dtype=np.uint8)
    aq[0, 0] = 2  # code 2 = +1.0 at column 0 of row 0
    wq = np.zeros((n, k // 2), dtype=np.uint8)
    wq[:, 0] = 2
    as_ = np.full(oracle.scale_bytes(1, k), 0x38, dtype=np.uint8)  # UE4M3 0x38 = 1.0
    ws = np.full(oracle.scale_bytes(n, k), 0x38, dtype=np.uint8)
    ga, gw = 257.0 / 256.0, 1.0
    bias = np.array([0x0000, 0x0001, 0x8001, 0x2F80, 0xAF80, 0x3B80, 0xBB80, 0x8000,
                     0x3F80, 0xBF80, 0x0000, 0x0001, 0x0000, 0x0001, 0x0000, 0x0001], dtype=np.uint16)
    d1, _ = oracle.gemm_rows_ex(aq, as_, 1, ga, wq, ws, n, gw, k, [0, 1], bias=bias)
    x = Fraction(257, 256)
    for j in range(n):
        assert d1[0, j] == exact.rn_bf16_bits(x + exact.bf16_value(int(bias[j]))), j
        assert d1[1, j] == exact.rn_bf16_bits(exact.bf16_value(int(bias[j]))) or (bias[j] == 0x8000 and d1[1, j] == 0)
    assert d1[0, 0] == 0x3F80 and d1[0, 1] == 0x3F81 and d1[0, 2] == 0x3F80
