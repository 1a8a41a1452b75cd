"""GPU parity of the block-scaled GEMM (stage G) and of the whole FC2 path against the
CPU oracle, through the C ABI.

The producer output is checked bit-exact first (so both sides multiply the same
bytes); the GEMM output is checked within the tolerance stated in tests/parity.py
on every row for small shapes, and on seeded sampled rows plus every padding row
at full size.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_path(w, device, rows_sample, seed):
    """Producer (SwiGLU or plain) + weight quantization + GEMM on the GPU; oracle on the
    same inputs; returns the GEMM statistics."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    _say(f"[path] {w.name}: m={w.m} n={w.n} k={w.k}")
    acts = w.activations()
    W = w.weight()
    a, aq, as_, ga = parity.run_quantize(acts[0], acts[1] if w.swiglu else None, device)
    wt, wq, ws, gw = parity.run_quantize(W, None, device)
    rq, rs, rg = oracle.quantize(acts[0], acts[1] if w.swiglu else None)
    assert (aq == rq).all() and (as_ == rs).all() and ga == rg, f"{w.name}: activation bytes differ"
    rwq, rws, rgw = oracle.quantize(W)
    assert (wq == rwq).all() and (ws == rws).all() and gw == rgw, f"{w.name}: weight bytes differ"
    del acts
    _say(f"[path] {w.name}: GEMM")
    d = nv.nvfp4_gemm_bf16out(a, wt)
    torch.cuda.synchronize()
    rows = np.arange(w.m_pad) if rows_sample is None else parity.sample_rows(w.m, w.m_pad, rows_sample, seed)
    got = parity.tensor_bits(d[torch.from_numpy(rows).to(device)])
    ref = oracle.gemm_rows(rq, rs, w.m, rg, rwq, rws, w.n, rgw, w.k, rows)
    st = parity.assert_gemm_close(got, ref, w.name)
    pad = rows >= w.m
    assert (got[pad] == 0).all(), "padding rows must be +0"
    _say(f"[path] {w.name}: {st}")
    return d, st


def test_tiny_full(gpu):
    d, st = run_path(synth.TINY, gpu, None, 0)
    assert st["checked"] == 256 * 512


@pytest.mark.parametrize("m,n,k", [(16, 16, 64), (48, 32, 128), (100, 272, 192), (300, 512, 320),
                                   (257, 256, 1024), (513, 528, 448)])
def test_small_shapes(gpu, m, n, k):
    """Tails in M (padding rows, partial 256-row tiles), N (n % 256 != 0) and K
    (k % 128 == 64: a half K step)."""
    w = synth.Workload(f"shape_{m}x{n}x{k}", m=m, n=n, k=k, seed=m + n + k, swiglu=True)
    run_path(w, gpu, None, 0)


def test_tail_quarter_tiles(gpu):
    """When the last round of 256 x 256 tiles would hold at most a quarter of the CUs'
    worth, those tiles run as 128 x 128 quarters. The shape is chosen from the
    device's CU count so that the split happens, with an M tail (quarters wholly and
    partly past m_padded), an N tail and a half K step inside the quarters; every
    output element is compared."""
    import torch
    cu = torch.cuda.get_device_properties(gpu).multi_processor_count
    tiles_n = 17
    tiles_m = (cu + cu // 16 + tiles_n - 1) // tiles_n
    tiles = tiles_m * tiles_n
    tail = tiles % cu
    assert tiles > cu and 0 < tail and 4 * tail <= cu, (cu, tiles_m, tiles_n)
    m = tiles_m * 256 - 96              # m_pad = m: the last quarter row is partly past it
    n = tiles_n * 256 - 16
    w = synth.Workload(f"tail_quarters_{m}x{n}", m=m, n=n, k=320, seed=17, swiglu=True)
    _say(f"[tail] {cu} CUs: {tiles} tiles, {tail} run as quarters")
    run_path(w, gpu, None, 0)


def test_persistent_tiles(gpu):
    """The plain GEMM runs its whole tiles with persistent workgroups (a multiple of 8
    of them, one per CU) when there are more whole tiles than that; each walks about
    three tiles here, loading the next tile while the last one's epilogue runs, and the
    leftover tiles run as quarters. M and N tails and a half K step; every output
    element is compared."""
    import torch
    cu = torch.cuda.get_device_properties(gpu).multi_processor_count
    persist = cu - cu % 8
    tiles_n = 17
    tiles_m = (3 * cu + cu // 16 + tiles_n - 1) // tiles_n
    tiles = tiles_m * tiles_n
    tail = tiles % cu
    big = tiles - tail if (0 < tail and 4 * tail <= cu) else tiles
    assert big > persist and big < tiles, (cu, tiles, tail)
    m = tiles_m * 256 - 96
    n = tiles_n * 256 - 16
    w = synth.Workload(f"persistent_{m}x{n}", m=m, n=n, k=192, seed=23, swiglu=True)
    _say(f"[persistent] {cu} CUs: {tiles} tiles, {big} whole over {persist} workgroups, {tiles - big} as quarters")
    run_path(w, gpu, None, 0)


def test_subnormal_scales(gpu):
    """Operands whose block scales are UE4M3 subnormals (E = 0) on both sides."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, n, k = 128, 128, 256
    x = synth.normal_bf16(m, k, seed=21, tag=4, sigma=1e-3)
    x[0, 0] = 0x4528  # 2688: g_a = 1, most blocks then take scale bytes 1..7
    wt = synth.normal_bf16(n, k, seed=21, tag=5, sigma=1e-3)
    wt[1, 1] = 0x4528
    a, aq, as_, ga = parity.run_quantize(x, None, gpu)
    w_, wq, ws, gw = parity.run_quantize(wt, None, gpu)
    assert ((as_ >= 1) & (as_ <= 7)).sum() > 100 and ((ws >= 1) & (ws <= 7)).sum() > 100
    d = nv.nvfp4_gemm_bf16out(a, w_)
    torch.cuda.synchronize()
    ref = oracle.gemm_rows(aq, as_, m, ga, wq, ws, n, gw, k, np.arange(m))
    parity.assert_gemm_close(parity.tensor_bits(d), ref, "subnormal scales")


def test_gemm_deterministic_and_prefix_invariant(gpu):
    """Bitwise identical on repeat, and the rows shared by a shorter m_padded over the
    same packed activation are bitwise identical (no dependence on the row count)."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    w = synth.Workload("prefix", m=1000, n=512, k=1024, seed=3, swiglu=True)
    gate, up = w.activations()
    a, *_ = parity.run_quantize(gate, up, gpu)
    wt, *_ = parity.run_quantize(w.weight(), None, gpu)
    d1 = nv.nvfp4_gemm_bf16out(a, wt)
    d2 = nv.nvfp4_gemm_bf16out(a, wt)
    short = nv.Nvfp4Tensor(qdata=a.qdata[:512], scales=a.scales, global_scale=a.global_scale, rows=512, k=a.k)
    d3 = nv.nvfp4_gemm_bf16out(short, wt)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)
    assert torch.equal(d1[:512], d3)


@pytest.mark.parametrize("name", ["mid_fc2_slice", "qkv", "attn_out", "fc1", "qkv_pages"])
def test_large_configs(gpu, name):
    """Configs 2 and 4 (and the pages' QKV width): 4,096 seeded rows, the tile-boundary
    rows and every padding row."""
    _, st = run_path(synth.BY_NAME[name], gpu, parity.PARITY_ROWS, 17)
    assert st["checked"] >= parity.PARITY_ROWS * synth.BY_NAME[name].n


def test_canonical_fc2(gpu):
    _, st = run_path(synth.FC2, gpu, parity.PARITY_ROWS, 440420)
    assert st["checked"] >= parity.PARITY_ROWS * synth.FC2.n


@pytest.mark.parametrize("m", synth.RAGGED_M)
def test_ragged_m(gpu, m):
    """Config 5: each ragged M with 4,096 seeded rows, the tile-boundary rows, the last
    64 logical rows and every padding row (the pages' row-shape gate found two
    differing bf16 elements in a whole output at some of these M)."""
    w = [r for r in synth.RAGGED if r.m == m][0]
    _, st = run_path(w, gpu, parity.PARITY_ROWS, m)
    assert st["checked"] >= parity.PARITY_ROWS * w.n
