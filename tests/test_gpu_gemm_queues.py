"""GPU checks of the plain GEMM's run-time tile queues: every tile is computed exactly
once whatever order the workgroups take them in, each launch leaves its queue set
cleared for the launch that reuses it, and launches in flight together on two streams
use separate sets. Outputs are compared with the CPU oracle on every element, and
with each other bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu

QUEUE_SETS = 64  # sets per device, taken round-robin by the plain GEMM's launches


def _say(msg):
    print(msg, flush=True)


def _shape(cu, rounds_times_16, tiles_n=17):
    """tiles_m for roughly rounds_times_16 / 16 rounds of tiles over the CUs."""
    return (rounds_times_16 * cu // 16 + tiles_n - 1) // tiles_n


def _operands(w, device):
    import nvfp4_block_scaled_swiglu_amd as nv  # noqa: F401
    gate, up = w.activations()
    a, aq, as_, ga = parity.run_quantize(gate, up, device)
    wt, wq, ws, gw = parity.run_quantize(w.weight(), None, device)
    rq, rs, rg = oracle.quantize(gate, up)
    assert (aq == rq).all() and (as_ == rs).all() and ga == rg
    rwq, rws, rgw = oracle.quantize(w.weight())
    assert (wq == rwq).all() and (ws == rws).all() and gw == rgw
    return a, wt, (rq, rs, rg, rwq, rws, rgw)


def _check_all_rows(d, w, ref_ops, name):
    rq, rs, rg, rwq, rws, rgw = ref_ops
    rows = np.arange(w.m_pad)
    got = parity.tensor_bits(d)
    ref = oracle.gemm_rows(rq, rs, w.m, rg, rwq, rws, w.n, rgw, w.k, rows)
    st = parity.assert_gemm_close(got, ref, name)
    assert (got[rows >= w.m] == 0).all()
    return st


def test_queue_sets_cleared_across_launches(gpu):
    """Two full cycles of the queue sets plus a few: a persistent launch whose tiles
    are mostly taken at run time (K = 512: the take is issued in the first K step),
    with a quarter tail. The first output is compared with the oracle on every
    element; every later launch, which reuses a set an earlier launch cleared, must
    match it bit for bit."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    cu = torch.cuda.get_device_properties(gpu).multi_processor_count
    tiles_m = _shape(cu, 33)
    tiles = tiles_m * 17
    tail = tiles % cu
    assert tiles > 2 * cu and 0 < tail and 4 * tail <= cu, (cu, tiles)
    w = synth.Workload(f"queues_{tiles_m * 256 - 96}x{17 * 256 - 16}", m=tiles_m * 256 - 96, n=17 * 256 - 16, k=512,
                       seed=41, swiglu=True)
    _say(f"[queues] {cu} CUs: {tiles} tiles, {tail} as quarters, {2 * QUEUE_SETS + 3} launches")
    a, wt, ref_ops = _operands(w, gpu)
    d0 = nv.nvfp4_gemm_bf16out(a, wt)
    torch.cuda.synchronize()
    st = _check_all_rows(d0, w, ref_ops, w.name)
    _say(f"[queues] first launch: {st}")
    d = torch.empty_like(d0)
    for i in range(2 * QUEUE_SETS + 2):
        d.fill_(-1)
        nv.nvfp4_gemm_bf16out(a, wt, out=d)
        if i % 16 == 15 or i == 2 * QUEUE_SETS + 1:
            torch.cuda.synchronize()
            assert torch.equal(d, d0), f"launch {i + 2} differs"
    torch.cuda.synchronize()
    assert torch.equal(d, d0)


def test_half_round_of_quarters(gpu):
    """A last round of whole tiles more than a quarter full: half a round of tiles
    runs as quarters after the whole tiles. K = 320 gives three K steps (the take in the
    first, then the two peeled steps, the last a half step); M and N tails; every
    element is compared with the oracle."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    cu = torch.cuda.get_device_properties(gpu).multi_processor_count
    tiles_m = _shape(cu, 40)
    tiles = tiles_m * 17
    tail = tiles % cu
    persist = cu - cu % 8
    assert 4 * tail > cu and tiles - persist // 2 > persist, (cu, tiles, tail)
    w = synth.Workload(f"half_round_{tiles_m * 256 - 96}x{17 * 256 - 16}", m=tiles_m * 256 - 96, n=17 * 256 - 16,
                       k=320, seed=43, swiglu=True)
    _say(f"[half round] {cu} CUs: {tiles} tiles, {persist // 2} as quarters")
    a, wt, ref_ops = _operands(w, gpu)
    d = nv.nvfp4_gemm_bf16out(a, wt)
    torch.cuda.synchronize()
    _say(f"[half round] {_check_all_rows(d, w, ref_ops, w.name)}")


def test_two_streams_in_flight(gpu):
    """Two plain GEMMs launched on two streams without waiting for each other (each
    launch takes its own queue set) give the same bits as the same GEMMs run one at a
    time."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    cu = torch.cuda.get_device_properties(gpu).multi_processor_count
    ws = [synth.Workload("streams_a", m=_shape(cu, 24) * 256 - 32, n=17 * 256, k=384, seed=45, swiglu=True),
          synth.Workload("streams_b", m=_shape(cu, 20) * 256, n=17 * 256 - 48, k=256, seed=47, swiglu=True)]
    ops = []
    for w in ws:
        gate, up = w.activations()
        a, *_ = parity.run_quantize(gate, up, gpu)
        wt, *_ = parity.run_quantize(w.weight(), None, gpu)
        ops.append((a, wt))
    alone = [nv.nvfp4_gemm_bf16out(a, wt) for a, wt in ops]
    torch.cuda.synchronize()
    outs = [torch.full_like(x, -1) for x in alone]
    streams = [torch.cuda.Stream(gpu), torch.cuda.Stream(gpu)]
    _say("[streams] two launches in flight, three rounds")
    for _ in range(3):
        for s, (a, wt), o in zip(streams, ops, outs):
            s.wait_stream(torch.cuda.current_stream(gpu))
            with torch.cuda.stream(s):
                o.fill_(-1)
                nv.nvfp4_gemm_bf16out(a, wt, out=o)
        torch.cuda.synchronize()
        for o, x in zip(outs, alone):
            assert torch.equal(o, x)
