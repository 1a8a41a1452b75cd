"""Pins for the oracle's SwiGLU-pair GEMM (step O14): the FC1 projection whose weight
rows interleave gate and up channels in chunks of 8, split back into gate and up,
with the row maxima of |RN_bf16(silu_bf16(gate) * up)| - the amax the FC2 producer
needs, emitted by the stage that writes gate and up (the component-2 summary's
conclusions put the global-scale dependency at this boundary).

The split is pinned in closed form with one-hot weight rows, and the maxima by the
already pinned O1-O2 applied to the returned gate and up.
"""
import numpy as np

import oracle
import synth


def quantize_pair(m, n_half, k, seed):
    x = synth.normal_bf16(m, k, seed=seed, tag=1, sigma=1.0)
    wg = synth.normal_bf16(n_half, k, seed=seed, tag=2, sigma=0.05)
    wu = synth.normal_bf16(n_half, k, seed=seed, tag=3, sigma=0.05)
    w = np.empty((2 * n_half, k), dtype=np.uint16)
    for c in range(n_half // 8):  # interleave written out row by row
        w[16 * c:16 * c + 8] = wg[8 * c:8 * c + 8]
        w[16 * c + 8:16 * c + 16] = wu[8 * c:8 * c + 8]
    aq, as_, ga = oracle.quantize(x)
    wq, ws, gw = oracle.quantize(w)
    return x, w, (aq, as_, ga, wq, ws, gw)


def test_interleave_helper_matches_row_by_row():
    _, w, _ = quantize_pair(8, 32, 64, 1)
    wg = np.concatenate([w[16 * c:16 * c + 8] for c in range(4)])
    wu = np.concatenate([w[16 * c + 8:16 * c + 16] for c in range(4)])
    assert (oracle.interleave_swiglu_rows(wg, wu) == w).all()


def test_split_one_hot_closed_form():
    """Gate channel j reads input column j (weight 1.0), up channel j reads column j
    with weight 2.0: gate = a[:, j], up = 2 a[:, j] exactly, for the dequantized a."""
    m, n_half, k = 16, 32, 64
    x = synth.normal_bf16(m, k, seed=5, tag=1, sigma=1.0)
    aq, as_, ga = oracle.quantize(x)
    wg = np.zeros((n_half, k), np.uint16)
    wu = np.zeros((n_half, k), np.uint16)
    for j in range(n_half):
        wg[j, j] = 0x3F80  # 1.0
        wu[j, j] = 0x4000  # 2.0
    w = oracle.interleave_swiglu_rows(wg, wu)
    wq, ws, gw = oracle.quantize(w)
    gate, up, ymax = oracle.gemm_swiglu_rows(aq, as_, m, ga, wq, ws, n_half, gw, k, np.arange(m))
    plain = oracle.gemm_rows(aq, as_, m, ga, wq, ws, 2 * n_half, gw, k, np.arange(m))
    cols = np.arange(n_half)
    gate_cols = 16 * (cols // 8) + cols % 8
    assert (gate == plain[:, gate_cols]).all() and (up == plain[:, gate_cols + 8]).all()
    g = oracle.bf16_bits_to_f32(gate).astype(np.float64)
    u = oracle.bf16_bits_to_f32(up).astype(np.float64)
    assert np.array_equal(u, 2 * g)  # a doubling is exact in bf16
    assert (np.abs(g) > 0).mean() > 0.9


def test_row_maxima_are_swiglu_of_the_outputs():
    m, n_half, k = 24, 64, 128
    _, _, (aq, as_, ga, wq, ws, gw) = quantize_pair(m, n_half, k, 7)
    bias = synth.normal_bf16(1, 2 * n_half, seed=7, tag=4, sigma=0.1)[0]
    rows = np.arange(oracle.padded_rows(m))
    gate, up, ymax = oracle.gemm_swiglu_rows(aq, as_, m, ga, wq, ws, n_half, gw, k, rows, bias=bias)
    want = np.zeros(rows.shape[0], np.float32)
    for i in range(rows.shape[0]):
        ys = [abs(float(oracle.bf16_bits_to_f32(np.array([oracle.swiglu_bf16(int(gate[i, j]), int(up[i, j]))]))[0]))
              for j in range(n_half)]
        want[i] = max(ys)
    assert np.array_equal(ymax, want)
    d1, _ = oracle.gemm_rows_ex(aq, as_, m, ga, wq, ws, 2 * n_half, gw, k, rows, bias=bias)
    cols = np.arange(n_half)
    gc = 16 * (cols // 8) + cols % 8
    assert (gate == d1[:, gc]).all() and (up == d1[:, gc + 8]).all()
