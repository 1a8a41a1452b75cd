"""GPU check of the matrix-core ceiling probe (a measurement aid beside the GEMM's
roofline, not a step of the method): every wave reports a positive cycle count and
a real-time span, and the clock they imply lies in the device's range."""
import pytest

pytestmark = pytest.mark.gpu


def test_ceiling_reports_every_wave(gpu):
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    print("[ceiling] 8 workgroups x 2048 iterations", flush=True)
    out = nv.nvfp4_mfma_ceiling(8, 2048)
    torch.cuda.synchronize()
    o = out.cpu()
    assert o.shape == (32, 2)
    assert (o[:, 0] > 0).all() and (o[:, 1] > 0).all()
    ghz = (o[:, 0].double() / (o[:, 1].double() / 100e6) / 1e9)
    assert ((ghz > 0.3) & (ghz < 4.0)).all(), ghz.tolist()


def test_hbm_stream_probe_writes_its_share(gpu):
    """The streaming probe reads every chunk and writes exactly the bytes it reports:
    chunk c fills dst[c * w, (c + 1) * w) with words derived from its own index, and the
    bytes after the written share keep their initial value."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    chunk = nv.lib().nvfp4_hbm_stream_chunk_bytes()
    chunks = 64
    src = torch.ones(chunks * chunk // 4, dtype=torch.int32, device=gpu)
    dst = torch.full((chunks * chunk // 4,), -7, dtype=torch.int32, device=gpu)
    print(f"[stream] {chunks} chunks of {chunk} B, write share 1/8", flush=True)
    written = nv.nvfp4_hbm_stream_ceiling(src, chunks * chunk, dst, chunks * chunk // 8)
    torch.cuda.synchronize()
    assert written == chunks * chunk // 8
    d = dst.cpu().view(-1, 4)  # 16-byte pieces: (xor, piece index, chunk index, 0)
    per = chunk // 8 // 16
    pieces = d[: chunks * per]
    assert (pieces[:, 1] == torch.arange(chunks * per) % per).all()
    assert (pieces[:, 2] == torch.arange(chunks * per) // per).all()
    assert (pieces[:, 3] == 0).all()
    assert (dst.cpu()[chunks * per * 4:] == -7).all()


def test_gemm_clock_stamps_leave_the_output_unchanged(gpu):
    """The clock-stamped GEMM (a measurement aid) writes the same output as
    nvfp4_gemm_bf16out, bit for bit, and every persistent workgroup's stamps give a
    clock in the device's range."""
    import torch
    import nvfp4_block_scaled_swiglu_amd as nv
    import synth
    from tests import parity
    cu = torch.cuda.get_device_properties(gpu).multi_processor_count
    w = synth.Workload("clock", m=3 * 1024, n=1024, k=512, seed=31, swiglu=True)  # 48 tiles
    gate, up = w.activations()
    a, *_ = parity.run_quantize(gate, up, gpu)
    wt, *_ = parity.run_quantize(w.weight(), None, gpu)
    print(f"[clock] {w.m}x{w.n}x{w.k}", flush=True)
    d0 = nv.nvfp4_gemm_bf16out(a, wt)
    d1 = torch.empty_like(d0)
    clk = torch.zeros((1024, 2), dtype=torch.int64, device=gpu)
    nv.nvfp4_gemm_bf16out_clock(a, wt, d1, clk)
    torch.cuda.synchronize()
    assert torch.equal(d0, d1)
    c = clk.cpu()
    used = c[:, 1] > 0
    assert used.sum() >= min(48, cu - cu % 8)
    ghz = c[used, 0].double() / (c[used, 1].double() / 100e6) / 1e9
    assert ((ghz > 0.3) & (ghz < 4.0)).all(), ghz.tolist()
