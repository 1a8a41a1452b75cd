"""Host-side checks of the C-ABI boundary (no GPU needed): the shared library loads,
exports every symbol include/nvfp4.h declares, its size functions agree with the
oracle's geometry, and argument validation returns the documented status codes
before anything touches a device."""
import ctypes
import os
import re
import subprocess

import pytest

import nvfp4_block_scaled_swiglu_amd as nv
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert "nvfp4_quantize_swiglu" in names and "nvfp4_gemm_bf16out" in names
    lib = nv.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", nv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (nvfp4_[a-z0-9_]+)", out))
    assert set(names) <= exported
    # the binding declares exactly the header's functions
    assert set(nv.SIGNATURES) == set(names)


def test_library_is_gfx950_only():
    """The embedded device code objects target gfx950 and nothing else."""
    out = subprocess.run(["strings", nv.LIB_PATH], capture_output=True, text=True).stdout
    targets = set(re.findall(r"amdgcn-amd-amdhsa--(gfx[0-9a-f]+)", out))
    assert targets == {"gfx950"}, targets


@pytest.mark.parametrize("rows,k", [(0, 64), (1, 64), (16, 1024), (37810, 14336), (37711, 14336), (5376, 14336),
                                    (16128, 5376), (28672, 5376), (37810, 7168), (130, 192)])
def test_sizes_match_oracle_geometry(rows, k):
    assert nv.nvfp4_padded_rows(rows) == oracle.padded_rows(rows)
    assert nv.nvfp4_qdata_bytes(rows, k) == oracle.qdata_bytes(rows, k)
    assert nv.nvfp4_scale_bytes(rows, k) == oracle.scale_bytes(rows, k)
    assert nv.nvfp4_scale_rows(rows) == oracle.scale_rows(rows)
    assert nv.nvfp4_scale_cols(k) == oracle.scale_cols(k)


def test_size_functions_reject_negative():
    assert nv.nvfp4_padded_rows(-1) == -1
    assert nv.nvfp4_qdata_bytes(-1, 64) == -1
    assert nv.nvfp4_quantize_workspace_bytes() == 16384


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced: validation fails first


def call_quant(**kw):
    args = dict(x=FAKE, ld=64, rows=16, k=64, q=FAKE, s=FAKE, g=FAKE, ws=FAKE)
    args.update(kw)
    return nv.lib().nvfp4_quantize(args["x"], args["ld"], args["rows"], args["k"], args["q"], args["s"],
                                   args["g"], args["ws"], None)


def call_swiglu(**kw):
    args = dict(g_=FAKE, ldg=64, u=FAKE, ldu=64, m=16, k=64, q=FAKE, s=FAKE, g=FAKE, ws=FAKE)
    args.update(kw)
    return nv.lib().nvfp4_quantize_swiglu(args["g_"], args["ldg"], args["u"], args["ldu"], args["m"], args["k"],
                                          args["q"], args["s"], args["g"], args["ws"], None)


def call_gemm(**kw):
    args = dict(aq=FAKE, as_=FAKE, ga=FAKE, wq=FAKE, ws=FAKE, gw=FAKE, d=FAKE, m=16, n=16, k=64)
    args.update(kw)
    return nv.lib().nvfp4_gemm_bf16out(args["aq"], args["as_"], args["ga"], args["wq"], args["ws"], args["gw"],
                                       args["d"], args["m"], args["n"], args["k"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(q=None), 1), (dict(s=None), 1), (dict(g=None), 1),
    (dict(ws=None), 4), (dict(rows=-1), 1), (dict(k=0), 1), (dict(k=96, ld=96), 2),
    (dict(ld=32), 1), (dict(ld=68), 3), (dict(x=FAKE + 8), 3), (dict(q=FAKE + 4), 3),
    (dict(g=FAKE + 2), 3),
])
def test_quantize_validation(kw, status):
    assert call_quant(**kw) == status
    assert nv.lib().nvfp4_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(u=None), 1), (dict(g_=None), 1), (dict(ldu=16), 1), (dict(ldg=68), 3), (dict(u=FAKE + 2), 3),
    (dict(k=32, ldg=32, ldu=32), 2),
])
def test_swiglu_validation(kw, status):
    assert call_swiglu(**kw) == status


def call_swiglu_amax(**kw):
    args = dict(g_=FAKE, ldg=64, u=FAKE, ldu=64, m=16, k=64, a=FAKE, q=FAKE, s=FAKE, g=FAKE)
    args.update(kw)
    return nv.lib().nvfp4_quantize_swiglu_amax(args["g_"], args["ldg"], args["u"], args["ldu"], args["m"],
                                               args["k"], args["a"], args["q"], args["s"], args["g"], None)


def call_quant_amax(**kw):
    args = dict(x=FAKE, ld=64, rows=16, k=64, a=FAKE, q=FAKE, s=FAKE, g=FAKE)
    args.update(kw)
    return nv.lib().nvfp4_quantize_amax(args["x"], args["ld"], args["rows"], args["k"], args["a"], args["q"],
                                        args["s"], args["g"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=None), 1), (dict(a=FAKE + 2), 3), (dict(u=None), 1), (dict(q=None), 1), (dict(k=32, ldg=32, ldu=32), 2),
    (dict(ldu=16), 1), (dict(ldg=68), 3), (dict(s=FAKE + 4), 3), (dict(m=-1), 1),
])
def test_swiglu_amax_validation(kw, status):
    """The single-read producer validates like the two-pass one; its amax pointer
    must be non-null and 4-byte aligned (an amax at FAKE + 4 is fine)."""
    assert call_swiglu_amax(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(a=None), 1), (dict(a=FAKE + 1), 3), (dict(x=None), 1), (dict(g=None), 1), (dict(k=96, ld=96), 2),
])
def test_quantize_amax_validation(kw, status):
    assert call_quant_amax(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(aq=None), 1), (dict(d=None), 1), (dict(ga=None), 1), (dict(n=0), 1), (dict(m=-16), 1),
    (dict(m=8), 2), (dict(n=24), 2), (dict(k=96), 2), (dict(d=FAKE + 8), 3), (dict(gw=FAKE + 1), 3),
    (dict(m=1 << 22, k=1 << 12), 2),
])
def test_gemm_validation(kw, status):
    assert call_gemm(**kw) == status


def call_modulate(**kw):
    args = dict(x=FAKE, ld=64, rows=16, k=64, sc=FAKE, sh=FAKE, q=FAKE, s=FAKE, g=FAKE, ws=FAKE)
    args.update(kw)
    return nv.lib().nvfp4_quantize_modulate(args["x"], args["ld"], args["rows"], args["k"], args["sc"], args["sh"],
                                            args["q"], args["s"], args["g"], args["ws"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(sc=None), 1), (dict(sh=None), 1), (dict(sc=FAKE + 2), 3), (dict(sh=FAKE + 8), 3), (dict(ws=None), 4),
    (dict(x=None), 1), (dict(k=96, ld=96), 2),
])
def test_modulate_validation(kw, status):
    assert call_modulate(**kw) == status


def call_fused(**kw):
    args = dict(aq=FAKE, as_=FAKE, ga=FAKE, wq=FAKE, ws=FAKE, gw=FAKE, d=FAKE, m=16, n=16, k=64, b=None, g=None,
                r=None)
    args.update(kw)
    return nv.lib().nvfp4_gemm_bf16out_fused(args["aq"], args["as_"], args["ga"], args["wq"], args["ws"],
                                             args["gw"], args["d"], args["m"], args["n"], args["k"], args["b"],
                                             args["g"], args["r"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=FAKE), 1), (dict(b=FAKE + 8), 3), (dict(g=FAKE + 2, r=FAKE), 3), (dict(r=FAKE + 4), 3),
    (dict(d=None), 1), (dict(m=8), 2), (dict(k=96), 2),
])
def test_fused_gemm_validation(kw, status):
    """The fused GEMM validates like the plain one; a gate needs a residual, and bias,
    gate and residual must be 16-byte aligned."""
    assert call_fused(**kw) == status


def call_pair(**kw):
    args = dict(aq=FAKE, as_=FAKE, ga=FAKE, wq=FAKE, ws=FAKE, gw=FAKE, g=FAKE, u=FAKE, m=16, nh=16, k=64, b=None,
                am=None, ar=16)
    args.update(kw)
    return nv.lib().nvfp4_gemm_swiglu_pair(args["aq"], args["as_"], args["ga"], args["wq"], args["ws"], args["gw"],
                                           args["g"], args["u"], args["m"], args["nh"], args["k"], args["b"],
                                           args["am"], args["ar"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(nh=12), 2), (dict(nh=0), 2), (dict(u=None), 1), (dict(g=None), 1), (dict(am=FAKE + 2), 3),
    (dict(ar=17), 1), (dict(ar=-1), 1), (dict(u=FAKE + 8), 3), (dict(b=FAKE + 4), 3),
])
def test_swiglu_pair_validation(kw, status):
    assert call_pair(**kw) == status


def test_silu_validation():
    assert nv.lib().nvfp4_silu_bf16(None, None, -1, None) == 1
    assert nv.lib().nvfp4_silu_bf16(None, FAKE, 4, None) == 1
    assert nv.lib().nvfp4_silu_bf16(FAKE + 1, FAKE, 4, None) == 3


def test_mfma_ceiling_validation():
    l = nv.lib()
    assert l.nvfp4_mfma_ceiling_out_bytes(3) == 3 * 4 * 16
    assert l.nvfp4_mfma_ceiling_out_bytes(0) == 0
    assert l.nvfp4_mfma_ceiling(0, 10, FAKE, 1 << 20, None) == 1
    assert l.nvfp4_mfma_ceiling(65537, 10, FAKE, 1 << 30, None) == 1
    assert l.nvfp4_mfma_ceiling(4, 0, FAKE, 1 << 20, None) == 1
    assert l.nvfp4_mfma_ceiling(4, (1 << 24) + 1, FAKE, 1 << 20, None) == 1
    assert l.nvfp4_mfma_ceiling(4, 10, None, 1 << 20, None) == 1
    assert l.nvfp4_mfma_ceiling(4, 10, FAKE + 4, 1 << 20, None) == 3
    assert l.nvfp4_mfma_ceiling(4, 10, FAKE, 4 * 4 * 16 - 1, None) == 1


def test_status_strings():
    for s in range(7):
        assert nv.nvfp4_status_string(s) not in ("", "unknown status")
    assert nv.nvfp4_status_string(99) == "unknown status"


def test_binding_raises_on_error():
    with pytest.raises(nv.Nvfp4Error) as ei:
        nv._call("nvfp4_gemm_bf16out", FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 64, None)
    assert ei.value.status == 2
    assert nv.COUNTERS["nvfp4_gemm_bf16out"]["failures"] >= 1


def test_strict_and_fallback_dispatch():
    """Strict calls raise; non-strict calls return False and count a fallback with the
    status and detail kept; successes, fallbacks and failures add up to the attempts.
    (Validation fails before any device access, so no GPU is needed.)"""
    name = "nvfp4_gemm_bf16out"
    before = nv.dispatch_counters().get(name, {"attempts": 0, "successes": 0, "fallbacks": 0, "failures": 0})
    bad = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 64, None)  # m_padded % 16 != 0
    with pytest.raises(nv.Nvfp4Error):
        nv._call(name, *bad, strict=True)
    assert nv._call(name, *bad, strict=False) is False
    assert nv.LAST_FALLBACK[name][0] == 2 and "m_padded" in nv.LAST_FALLBACK[name][1]
    saved = nv.STRICT
    try:
        nv.set_strict(False)
        assert nv._call(name, *bad) is False
        nv.set_strict(True)
        with pytest.raises(nv.Nvfp4Error):
            nv._call(name, *bad)
    finally:
        nv.set_strict(saved)
    after = nv.dispatch_counters()[name]
    assert after["attempts"] - before["attempts"] == 4
    assert after["fallbacks"] - before["fallbacks"] == 2
    assert after["failures"] - before["failures"] == 2
    assert after["attempts"] == after["successes"] + after["fallbacks"] + after["failures"]


def test_strict_default_follows_environment():
    """NVFP4_STRICT=0 starts the binding non-strict; anything else (or unset) strict."""
    code = ("import nvfp4_block_scaled_swiglu_amd as nv; print(int(nv.STRICT))")
    env = dict(os.environ)
    outs = []
    for val in (None, "0", "1"):
        if val is None:
            env.pop("NVFP4_STRICT", None)
        else:
            env["NVFP4_STRICT"] = val
        r = subprocess.run([os.environ.get("PYTHON", "python"), "-c", code], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=120)
        outs.append(r.stdout.strip())
    assert outs == ["1", "0", "1"]


def test_valid_call_without_gpu_reports_no_device():
    """With valid arguments and no visible GPU the call reaches the device check and
    returns NVFP4_ERR_NO_DEVICE (nothing is launched)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert call_quant() == 5
    assert "device" in nv.lib().nvfp4_last_error().decode().lower()


def test_hbm_stream_ceiling_validation():
    l = nv.lib()
    chunk = l.nvfp4_hbm_stream_chunk_bytes()
    assert chunk == 16384
    assert l.nvfp4_hbm_stream_ceiling(None, chunk, FAKE, 0, None) == 1
    assert l.nvfp4_hbm_stream_ceiling(FAKE, 0, FAKE, 0, None) == 1
    assert l.nvfp4_hbm_stream_ceiling(FAKE, chunk + 16, FAKE, 0, None) == 1
    assert l.nvfp4_hbm_stream_ceiling(FAKE, chunk, FAKE, chunk + 16, None) == 1
    assert l.nvfp4_hbm_stream_ceiling(FAKE, chunk, FAKE, 8, None) == 1
    assert l.nvfp4_hbm_stream_ceiling(FAKE + 4, chunk, FAKE, 0, None) == 3


def test_noalloc_entry_validation():
    """The no-allocation producer validates like nvfp4_quantize_swiglu (no workspace
    argument) and, with valid arguments and no GPU, stops at the device check."""
    l = nv.lib()
    f = l.nvfp4_quantize_swiglu_noalloc
    assert f(None, 64, FAKE, 64, 16, 64, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, 64, FAKE, 64, 16, 96, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 64, FAKE, 64, 16, 64, FAKE + 8, FAKE, FAKE, None) == 3
    assert f(FAKE, 64, FAKE, 64, 16, 64, FAKE, FAKE, None, None) == 1
    import torch
    if not torch.cuda.is_available():
        assert f(FAKE, 64, FAKE, 64, 16, 64, FAKE, FAKE, FAKE, None) == 5


def test_gemm_clock_entry_validation():
    """The clock-stamped GEMM validates its clock buffer, then as nvfp4_gemm_bf16out."""
    f = nv.lib().nvfp4_gemm_bf16out_clock
    g = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 16, 64)
    assert f(*g, None, 4, None) == 1
    assert f(*g, FAKE, 0, None) == 1
    assert f(*g, FAKE + 4, 4, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 64, FAKE, 4, None) == 2
