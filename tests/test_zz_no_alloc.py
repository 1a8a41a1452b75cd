"""GPU check of nvfp4_quantize_swiglu_noalloc, the producer entry point that allocates
nothing (its absmax partials live in the library's fixed device scratch): through the
C ABI, its bytes equal those of nvfp4_quantize_swiglu (caller workspace) and of the
oracle, on two calls in a row, the second with a smaller input (fewer absmax
workgroups, so slots written by the first call stay in the scratch unread)."""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _one(nv, torch, device, m, k, seed):
    gate = synth.normal_bf16(m, k, seed=seed, tag=1, sigma=1.0)
    up = synth.normal_bf16(m, k, seed=seed, tag=2, sigma=1.0)
    g_t, u_t = parity.to_device_bf16(gate, device), parity.to_device_bf16(up, device)
    out = nv.empty_nvfp4(m, k, device)
    for t in (out.qdata, out.scales):
        t.fill_(0xA5)
    got = nv.nvfp4_quantize_swiglu_noalloc(g_t, u_t, out)
    ref = nv.nvfp4_quantize_swiglu(g_t, u_t)
    torch.cuda.synchronize()
    assert got is out
    assert torch.equal(got.qdata, ref.qdata) and torch.equal(got.scales, ref.scales)
    assert torch.equal(got.global_scale, ref.global_scale)
    rq, rs, rg = oracle.quantize(gate, up)
    assert (got.qdata.cpu().numpy() == rq).all() and (got.scales.cpu().numpy() == rs).all()
    assert float(got.global_scale.item()) == rg
    return float(rg)


def test_noalloc_matches_workspace_entry_twice(gpu):
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    nv.nvfp4_init()
    _say("[noalloc] call 1: 2048 x 4096 (every absmax workgroup busy)")
    g1 = _one(nv, torch, gpu, 2048, 4096, 61)
    _say("[noalloc] call 2: 100 x 512 (two absmax workgroups)")
    # a smaller tensor with a much smaller amax: a stale partial from call 1 would show
    g2 = _one(nv, torch, gpu, 100, 512, 62)
    assert g1 > 0 and g2 > 0
