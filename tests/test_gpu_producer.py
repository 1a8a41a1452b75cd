"""GPU parity of the producer (stage P) against the CPU oracle, through the C ABI.

QDATA, scale buffer and global scale must be bit-exact, padding included, on every
workload and edge case.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def check_quant(x_bits, up_bits, device, what, m=None):
    _say(f"[producer] {what}: shape {x_bits.shape} m={m}")
    _, qd, sc, g = parity.run_quantize(x_bits, up_bits, device, m=m)
    rq, rs, rg = oracle.quantize(x_bits, up_bits, m=m)
    assert np.float32(g).view(np.uint32) == np.float32(rg).view(np.uint32), f"{what}: g {g!r} != {rg!r}"
    assert qd.shape == rq.shape and sc.shape == rs.shape
    nq = int((qd != rq).sum())
    ns = int((sc != rs).sum())
    assert nq == 0 and ns == 0, f"{what}: {nq} QDATA bytes and {ns} scale bytes differ"
    return qd, sc, g


def test_silu_table_all_bf16_inputs(gpu):
    """The producer's silu on all 65,536 bf16 bit patterns equals the oracle's
    correctly rounded silu (finite inputs)."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).to(gpu)
    y = nv.nvfp4_silu_bf16(x).cpu().numpy().view(np.uint16)
    want = oracle.silu_table()
    finite = (np.arange(65536) & 0x7F80) != 0x7F80
    bad = np.nonzero((y != want) & finite)[0]
    assert bad.size == 0, [hex(b) for b in bad[:10]]


def test_tiny_config(gpu):
    w = synth.TINY
    gate, up = w.activations()
    check_quant(gate, up, gpu, "tiny swiglu")
    check_quant(w.weight(), None, gpu, "tiny weight")


@pytest.mark.parametrize("m,k", [(1, 64), (15, 64), (16, 128), (17, 192), (130, 320), (255, 1024), (300, 576),
                                 (1000, 14336), (3000, 5376)])
def test_edge_shapes(gpu, m, k):
    """Ragged rows (padding to 16 and to 128-row scale tiles), widths that do not fill
    a 512-column unit, and grids on both sides of the quantize launch's split into
    whole groups and halves (1,000 x 14,336: 1,792 groups, 256 of them whole; 3,000 x
    5,376: 2,112 groups with a half-filled last column segment)."""
    gate = synth.normal_bf16(m, k, seed=m, tag=1, sigma=1.0)
    up = synth.normal_bf16(m, k, seed=m, tag=2, sigma=1.0)
    check_quant(gate, up, gpu, f"swiglu m={m} k={k}")
    check_quant(gate, None, gpu, f"plain m={m} k={k}")


def test_empty_rows(gpu):
    """m = 0: no QDATA or scale bytes, g = 0."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    x = torch.zeros((16, 64), dtype=torch.bfloat16, device=gpu)
    t = nv.nvfp4_quantize(x, rows=0)
    t2 = nv.nvfp4_quantize_swiglu(x, x, m=0)
    torch.cuda.synchronize()
    assert t.qdata.numel() == 0 and t.scales.numel() == 0
    assert float(t.global_scale.item()) == 0.0 and float(t2.global_scale.item()) == 0.0


def test_strided_inputs(gpu):
    """Row strides larger than k, different for gate and up."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    m, k = 200, 384
    gate_full = synth.normal_bf16(m, k + 64, seed=5, tag=1, sigma=1.0)
    up_full = synth.normal_bf16(m, k + 128, seed=5, tag=2, sigma=1.0)
    g_t = parity.to_device_bf16(gate_full, gpu)[:, :k]
    u_t = parity.to_device_bf16(up_full, gpu)[:, :k]
    t = nv.nvfp4_quantize_swiglu(g_t, u_t)
    torch.cuda.synchronize()
    rq, rs, rg = oracle.quantize(np.ascontiguousarray(gate_full[:, :k]), np.ascontiguousarray(up_full[:, :k]))
    assert (t.qdata.cpu().numpy() == rq).all() and (t.scales.cpu().numpy() == rs).all()
    assert float(t.global_scale.item()) == rg


def test_zero_and_signed_zero(gpu):
    x = np.zeros((32, 128), dtype=np.uint16)
    x[3, 5] = 0x8000
    x[7, 100] = 0x8000
    qd, sc, g = check_quant(x, None, gpu, "zeros")
    assert g == 0.0 and (sc == 0).all()


def test_exact_ties(gpu):
    """Blocks whose elements sit exactly on E2M1 rounding midpoints: amax = 2.625 gives
    g = 2^-10, the amax block gets S = 448 and unit 0.4375; every other element is
    mid * 0.4375 for a midpoint mid (all representable in bf16)."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows, k = 64, 256
    x = np.zeros((rows, k), dtype=np.float32)
    rng = np.random.default_rng(0)
    for r in range(rows):
        for b in range(k // 16):
            blk = [6.0 * 0.4375] + [mids[int(i)] * 0.4375 for i in rng.integers(0, 7, 15)]
            blk = np.array(blk) * np.where(rng.random(16) < 0.5, -1.0, 1.0)
            x[r, b * 16:(b + 1) * 16] = blk
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert ((bits.astype(np.uint32) << 16).view(np.float32) == x).all()
    qd, sc, g = check_quant(bits, None, gpu, "exact ties")
    assert g == 2.0 ** -10


def test_subnormal_products_and_tiny_tensor(gpu):
    """silu(gate) * up below 2^-126 (rounded once from the exact product), inside a
    normal tensor and in a tensor whose absmax itself is subnormal."""
    m, k = 64, 256
    rng = np.random.default_rng(1)
    gate = synth.normal_bf16(m, k, seed=9, tag=1, sigma=1.0)
    up = synth.normal_bf16(m, k, seed=9, tag=2, sigma=1.0)
    # silu(-90) ~ -7.4e-38; times small up values gives fp32 subnormal products
    sel = rng.random((m, k)) < 0.3
    gate[sel] = 0xC2B4  # -90
    up[sel] = (rng.integers(0x3A00, 0x3C80, size=sel.sum())).astype(np.uint16)
    check_quant(gate, up, gpu, "subnormal products in a normal tensor")
    gate2 = np.full((m, k), 0xC2B4, dtype=np.uint16)
    up2 = (rng.integers(0x3800, 0x3C00, size=(m, k))).astype(np.uint16)
    check_quant(gate2, up2, gpu, "all products subnormal")


def test_extreme_magnitudes_plain(gpu):
    """Plain quantization across the bf16 range: subnormal block scales, huge amax."""
    m, k = 128, 512
    rng = np.random.default_rng(2)
    x = synth.normal_bf16(m, k, seed=11, tag=4, sigma=1.0)
    x[0, 0] = 0x7F7F  # bf16 max
    x[5, 17] = 0x0001  # smallest subnormal
    x[9, :64] = 0x3F80
    check_quant(x, None, gpu, "bf16 max amax")
    y = synth.normal_bf16(m, k, seed=12, tag=4, sigma=1e-3)
    y[3, 3] = 0x4528  # 2688
    check_quant(y, None, gpu, "subnormal block scales")


def test_workspace_reuse_and_determinism(gpu):
    """A zero-filled workspace, reused by back-to-back calls of different sizes and
    modes, gives identical bytes each time, equal to the oracle's, and each call leaves
    the workspace zero-filled again (its quantize launch clears the absmax slots that
    its absmax launch filled)."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    w = synth.TINY
    gate, up = w.activations()
    g_t, u_t = parity.to_device_bf16(gate, gpu), parity.to_device_bf16(up, gpu)
    ws = torch.zeros((nv.nvfp4_quantize_workspace_bytes(),), dtype=torch.uint8, device=gpu)

    def zero_after(out):
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, "workspace not left zero-filled"
        return out

    outs = [zero_after(nv.nvfp4_quantize_swiglu(g_t, u_t, workspace=ws)) for _ in range(2)]
    x_t = parity.to_device_bf16(w.weight(), gpu)
    wq = zero_after(nv.nvfp4_quantize(x_t, workspace=ws))
    small = zero_after(nv.nvfp4_quantize_swiglu(g_t[:20], u_t[:20], workspace=ws))
    outs.append(zero_after(nv.nvfp4_quantize_swiglu(g_t, u_t, workspace=ws)))
    for o in outs[1:]:
        assert torch.equal(o.qdata, outs[0].qdata) and torch.equal(o.scales, outs[0].scales)
        assert torch.equal(o.global_scale, outs[0].global_scale)
    rq, rs, rg = oracle.quantize(gate, up)
    assert (outs[0].qdata.cpu().numpy() == rq).all() and (outs[0].scales.cpu().numpy() == rs).all()
    assert float(outs[0].global_scale.item()) == rg
    rq, rs, rg = oracle.quantize(w.weight())
    assert (wq.qdata.cpu().numpy() == rq).all() and float(wq.global_scale.item()) == rg
    rq, rs, rg = oracle.quantize(gate[:20], up[:20])
    assert (small.qdata.cpu().numpy() == rq).all() and (small.scales.cpu().numpy() == rs).all()
    assert float(small.global_scale.item()) == rg


def test_many_calls_two_streams(gpu):
    """70 calls queued without waiting, more than the 64 counter sets the quantize
    launches rotate through, alternating two streams (each with its own workspace) and
    two shapes whose grids take few and many groups. Every result equals the oracle's,
    and both workspaces end zero-filled."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    w = synth.MID
    gate, up = w.activations()  # 4,096 x 14,336: 7,168 groups, past the 6,144 that need no take
    small_g, small_u = gate[:40, :1024], up[:40, :1024]  # 20 groups
    refs = [oracle.quantize(np.ascontiguousarray(gate), np.ascontiguousarray(up)),
            oracle.quantize(np.ascontiguousarray(small_g), np.ascontiguousarray(small_u))]
    ins = [(parity.to_device_bf16(gate, gpu), parity.to_device_bf16(up, gpu)),
           (parity.to_device_bf16(small_g, gpu), parity.to_device_bf16(small_u, gpu))]
    streams = [torch.cuda.Stream(device=gpu), torch.cuda.Stream(device=gpu)]
    wss = [torch.zeros((nv.nvfp4_quantize_workspace_bytes(),), dtype=torch.uint8, device=gpu) for _ in streams]
    torch.cuda.synchronize(gpu)
    outs = []
    for i in range(70):
        sel = (i // 2) % 2  # shape: large, large, small, small, ...
        s_i = i % 2         # stream
        with torch.cuda.stream(streams[s_i]):
            g_t, u_t = ins[sel]
            outs.append((sel, nv.nvfp4_quantize_swiglu(g_t, u_t, workspace=wss[s_i], stream=streams[s_i])))
    torch.cuda.synchronize(gpu)
    _say(f"[producer] 70 queued calls on two streams done")
    for ws in wss:
        assert int(ws.count_nonzero()) == 0, "workspace not left zero-filled"
    for i, (sel, o) in enumerate(outs):
        rq, rs, rg = refs[sel]
        assert (o.qdata.cpu().numpy() == rq).all() and (o.scales.cpu().numpy() == rs).all(), f"call {i}"
        assert float(o.global_scale.item()) == rg, f"call {i}"


def test_non_strict_failure_leaves_buffers(gpu):
    """A call that fails validation, made non-strict, returns None, counts a fallback
    and leaves the produced NVFP4 bytes and the output buffer as they were."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    w = synth.TINY
    gate, up = w.activations()
    a = nv.nvfp4_quantize_swiglu(parity.to_device_bf16(gate, gpu), parity.to_device_bf16(up, gpu))
    wt = nv.nvfp4_quantize(parity.to_device_bf16(w.weight(), gpu))
    torch.cuda.synchronize()
    snap = (a.qdata.clone(), a.scales.clone(), a.global_scale.clone())
    # the same bytes described with k = 96 (not a multiple of 64): the library refuses
    bad_a = nv.Nvfp4Tensor(qdata=a.qdata, scales=a.scales, global_scale=a.global_scale, rows=a.rows, k=96)
    bad_w = nv.Nvfp4Tensor(qdata=wt.qdata, scales=wt.scales, global_scale=wt.global_scale, rows=wt.rows, k=96)
    out = torch.full((a.padded_rows, wt.rows), 7.0, dtype=torch.bfloat16, device=gpu)
    before = nv.dispatch_counters().get("nvfp4_gemm_bf16out", {}).get("fallbacks", 0)
    assert nv.nvfp4_gemm_bf16out(bad_a, bad_w, out=out, strict=False) is None
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_gemm_bf16out(bad_a, bad_w, out=out, strict=True)
    torch.cuda.synchronize()
    assert nv.dispatch_counters()["nvfp4_gemm_bf16out"]["fallbacks"] == before + 1
    assert bool((out == 7.0).all())
    assert torch.equal(a.qdata, snap[0]) and torch.equal(a.scales, snap[1]) and torch.equal(a.global_scale, snap[2])
    # the fallback goes through the same, untouched bytes
    d = nv.nvfp4_gemm_bf16out(a, wt)
    torch.cuda.synchronize()
    assert d is not None and bool(torch.isfinite(d.float()).all())


@pytest.mark.parametrize("name", ["mid_fc2_slice", "qkv", "attn_out", "fc1"])
def test_large_configs(gpu, name):
    w = synth.BY_NAME[name]
    acts = w.activations()
    check_quant(acts[0], acts[1] if w.swiglu else None, gpu, name)


def test_canonical_fc2(gpu):
    w = synth.FC2
    gate, up = w.activations()
    qd, sc, g = check_quant(gate, up, gpu, "canonical fc2")
    assert qd.shape == (37824, 7168) and sc.size == 37888 * 896
    assert (qd[37810:] == 0).all()


@pytest.mark.parametrize("m", synth.RAGGED_M)
def test_ragged_m(gpu, m):
    w = [r for r in synth.RAGGED if r.m == m][0]
    gate, up = w.activations()
    check_quant(gate, up, gpu, w.name)
