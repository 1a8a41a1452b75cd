"""Pins for the oracle's buffer geometry and the 128-row by 4-scale-column tiled scale
layout (step O8), against the byte counts the pages print (tests/golden/fc2_footprint.json).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

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
    # the oracle's offsets on a grid sample
    off = np.vectorize(oracle.scale_offset, otypes=[np.int64])(
        np.broadcast_to(r, (rp, cp))[:: max(1, rp // 64), :: max(1, cp // 16)],
        np.broadcast_to(c, (rp, cp))[:: max(1, rp // 64), :: max(1, cp // 16)], cp)
    full = tiled_positions(rp, cp)  # the storage order stated as reshapes (below), no offset formula
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


# ---- the order inside a 128 x 4 tile, derived without the offset formula ----------------
#
# The component-2 summary names the layout only ("general 128-row by 4-scale-column
# tiled offset", key native_pack_validation.fix). The reading taken is the tiled layout
# documented publicly for block-scaled FP4 operands: the scale grid is cut into tiles of
# 128 rows x 4 scale columns, stored one after another with the row tiles outermost;
# inside a tile the 128 rows form 4 groups of 32, and the tile's bytes run over the row
# within its group (outermost), then the group, then the column (innermost), so that
# rows i, i+32, i+64, i+96 share one 16-byte chunk. The function below states that
# storage order as reshapes and one transpose of a grid of element ids, and inverts the
# resulting permutation; it contains no offset arithmetic of its own.

def tiled_positions(rp: int, cp: int) -> np.ndarray:
    """pos[r, c]: the byte of the scale buffer that holds scale (r, c)."""
    ids = np.arange(rp * cp, dtype=np.int64).reshape(rp, cp)
    # axes: row tile, row group (4), row within group (32), column tile, column (4)
    cut = ids.reshape(rp // 128, 4, 32, cp // 4, 4)
    stored = cut.transpose(0, 3, 2, 1, 4).reshape(-1)  # storage order, outermost first
    pos = np.empty(rp * cp, dtype=np.int64)
    pos[stored] = np.arange(rp * cp, dtype=np.int64)
    return pos.reshape(rp, cp)


def test_tiled_positions_structure():
    """Sanity of the derivation itself on one tile: the first bytes of the tile hold row 0
    columns 0-3, then rows 32, 64, 96; the second 16-byte chunk starts with row 1; the next
    tile along the columns starts at byte 512."""
    pos = tiled_positions(128, 8)
    assert [int(pos[r, c]) for r, c in ((0, 0), (0, 1), (0, 3), (32, 0), (64, 0), (96, 3))] == [0, 1, 3, 4, 8, 15]
    assert int(pos[1, 0]) == 16 and int(pos[31, 3]) == 31 * 16 + 3 and int(pos[127, 3]) == 511
    assert int(pos[0, 4]) == 512
    chunk = sorted(int(pos[r, c]) // 16 for r in (5, 37, 69, 101) for c in range(4))
    assert chunk == [5] * 16


@pytest.mark.parametrize("rows,k", [(256, 1024), (48, 96), (16, 64), (1, 64), (300, 448), (37824, 14336)])
def test_oracle_swizzle_equals_tiled_positions(rows, k):
    """The oracle's scale offset (step O8) against the permutation derived above, on
    every (row, column) of the padded grid (a row sample for the full FC2 grid)."""
    rp, cp = oracle.scale_rows(rows), oracle.scale_cols(k)
    pos = tiled_positions(rp, cp)
    rsel = np.arange(rp) if rp <= 512 else np.unique(np.concatenate(
        [np.arange(0, 256), np.arange(rp - 256, rp), np.random.default_rng(8).choice(rp, 256, replace=False)]))
    csel = np.arange(cp) if cp <= 64 else np.unique(np.concatenate(
        [np.arange(0, 16), np.arange(cp - 16, cp), np.random.default_rng(9).choice(cp, 32, replace=False)]))
    got = np.array([[oracle.scale_offset(int(r), int(c), cp) for c in csel] for r in rsel], dtype=np.int64)
    np.testing.assert_array_equal(got, pos[np.ix_(rsel, csel)])


def test_oracle_scale_buffer_through_tiled_positions():
    """The whole scale buffer the oracle writes, read back through the derived layout:
    every real byte is the block scale of its (row, block) (step O5, pinned separately by
    brute force), and every byte outside the real rows and columns is zero."""
    m, k = 200, 448  # padded rows 208 of 256 scale rows; 28 blocks of 28 scale columns
    x = synth.normal_bf16(m, k, seed=41, tag=9, sigma=1.0)
    qd, sc, g = oracle.quantize(x)
    rp, cp = oracle.scale_rows(m), oracle.scale_cols(k)
    grid = sc[tiled_positions(rp, cp)]
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bmax = np.abs(xf).reshape(m, k // 16, 16).max(axis=2)
    want = np.zeros((rp, cp), dtype=np.uint8)
    for r in range(m):
        for b in range(k // 16):
            want[r, b] = oracle.block_scale(float(bmax[r, b]), g)
    np.testing.assert_array_equal(grid, want)
