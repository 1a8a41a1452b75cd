"""Pins for the oracle's buffer geometry and the 128-row by 4-scale-column tiled scale
layout (step O8), against the byte counts the pages print (tests/golden/fc2_footprint.json).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fc2_footprint.json")))


def test_fc2_footprint_matches_pages():
    t = GOLDEN["fc2_traffic_attribution"]
    m, mp, n, k = t["m_logical"], t["m_descriptor"], t["n"], t["k"]
    assert oracle.padded_rows(m) == mp
    # nominal (unpadded-row) scale bytes, as the footprint table counts them
    a_bytes = oracle.qdata_bytes(m, k) + oracle.padded_rows(m) * (k // 16)
    w_bytes = oracle.qdata_bytes(n, k) + n * (k // 16)
    d_bytes = mp * n * 2
    assert a_bytes == t["activation_qdata_plus_scales"]
    assert w_bytes == t["weight_qdata_plus_scales"]
    assert d_bytes == t["padded_bf16_output"]
    assert a_bytes + w_bytes + d_bytes == t["total"]
    # request geometry of 128x128 output tiles over the 128-padded scale rows
    m_tiles = oracle.scale_rows(m) // 128
    assert m_tiles == t["weight_geometric_reuse"]
    assert m_tiles * w_bytes == t["requested_weight_bytes_128x128_tiles"]
    n_tiles = n // 128
    assert n_tiles * oracle.scale_rows(m) * (k // 2 + k // 16) == t["requested_activation_bytes_128x128_tiles"]


def test_scale_rows_are_padded_to_128():
    """The component-2 intermediate byte count decomposes exactly with scale rows padded
    to whole 128-row tiles (and not with 16-row padding)."""
    c = GOLDEN["component2_intermediates"]
    m = c["m_logical"]
    total = 0
    total16 = 0
    for k, n in c["projections_k_n"].values():
        base = m * k * 2 + oracle.qdata_bytes(m, k) + m * n * 2
        total += base + oracle.scale_bytes(m, k)
        total16 += base + oracle.padded_rows(m) * (k // 16)
    assert total == c["bytes"]
    assert total16 != c["bytes"]


@pytest.mark.parametrize("rows,k", [(37824, 14336), (256, 1024), (5376, 14336), (37824, 7168),
                                    (37824, 5376), (48, 96), (16, 16), (1, 64)])
def test_swizzle_is_a_tiled_bijection(rows, k):
    """Every (row, column) of the padded scale grid maps to a distinct byte of
    [0, R' * C'), and each 128-row x 4-column tile fills one contiguous 512-byte run,
    tiles in row-tile-major order."""
    rp = oracle.scale_rows(rows)
    cp = oracle.scale_cols(k)
    r = np.arange(rp, dtype=np.int64)[:, None]
    c = np.arange(cp, dtype=np.int64)[None, :]
    # vectorised evaluation of the oracle's offset, checked against its scalar form
    off = np.vectorize(oracle.scale_offset, otypes=[np.int64])(
        np.broadcast_to(r, (rp, cp))[:: max(1, rp // 64), :: max(1, cp // 16)],
        np.broadcast_to(c, (rp, cp))[:: max(1, rp // 64), :: max(1, cp // 16)], cp)
    full = ((r >> 7) * (cp // 4) + (c >> 2)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 3)
    np.testing.assert_array_equal(off, full[:: max(1, rp // 64), :: max(1, cp // 16)])
    flat = full.ravel()
    assert flat.min() == 0 and flat.max() == rp * cp - 1
    assert np.unique(flat).size == rp * cp
    tile = (r >> 7) * (cp // 4) + (c >> 2)
    assert ((full // 512) == tile).all()


def test_regression_widths_are_exact_tilings():
    for k in GOLDEN["regression_widths"]["widths"]:
        assert (k // 16) % 4 == 0
        assert oracle.scale_cols(k) == k // 16
