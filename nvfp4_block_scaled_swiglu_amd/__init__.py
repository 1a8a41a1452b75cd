"""MI355X (gfx950) NVFP4 SwiGLU producer and block-scaled GEMM - Python binding.

A thin ctypes layer over the C ABI in ``include/nvfp4.h`` (``libnvfp4.so``, built
in-tree by ``build.py``). Every step of the computation runs in the library's HIP
kernels; this module only marshals torch tensors (device memory) and the current
torch stream into the C calls, and allocates outputs with torch when the caller
does not pass them. There is no fallback computation: if the library is missing,
the first call raises ImportError; if a call fails it raises (strict, the default)
or returns None and counts a fallback (non-strict), leaving the caller's buffers as
they were.

Functions carry the C names:

* ``nvfp4_quantize_swiglu(gate, up)`` - fused SwiGLU -> NVFP4 producer
* ``nvfp4_quantize(x)``               - plain NVFP4 quantization (activations, weights)
* ``nvfp4_gemm_bf16out(a, w)``        - block-scaled GEMM, FP32 accumulation, BF16 out
* ``nvfp4_silu_bf16(x)``              - the producer's bf16 silu, elementwise (self-test)
* size helpers ``nvfp4_padded_rows``, ``nvfp4_qdata_bytes``, ``nvfp4_scale_bytes``, ...
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

NVFP4_OK = 0
STATUS_NAMES = {
    0: "NVFP4_OK",
    1: "NVFP4_ERR_INVALID_ARG",
    2: "NVFP4_ERR_UNSUPPORTED_SHAPE",
    3: "NVFP4_ERR_MISALIGNED",
    4: "NVFP4_ERR_WORKSPACE",
    5: "NVFP4_ERR_NO_DEVICE",
    6: "NVFP4_ERR_LAUNCH",
}

# Every symbol include/nvfp4.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
SIGNATURES = {
    "nvfp4_padded_rows": (_I64, [_I64]),
    "nvfp4_scale_rows": (_I64, [_I64]),
    "nvfp4_scale_cols": (_I64, [_I64]),
    "nvfp4_qdata_bytes": (_I64, [_I64, _I64]),
    "nvfp4_scale_bytes": (_I64, [_I64, _I64]),
    "nvfp4_quantize_workspace_bytes": (_I64, []),
    "nvfp4_init": (_INT, []),
    "nvfp4_quantize_swiglu": (_INT, [_P, _I64, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "nvfp4_quantize_swiglu_noalloc": (_INT, [_P, _I64, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_quantize": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "nvfp4_quantize_modulate": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "nvfp4_quantize_swiglu_amax": (_INT, [_P, _I64, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "nvfp4_quantize_amax": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "nvfp4_gemm_bf16out": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "nvfp4_gemm_bf16out_clock": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "nvfp4_gemm_bf16out_fused": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_gemm_swiglu_pair": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64, _P]),
    "nvfp4_silu_bf16": (_INT, [_P, _P, _I64, _P]),
    "nvfp4_mfma_ceiling_out_bytes": (_I64, [_I64]),
    "nvfp4_mfma_ceiling": (_INT, [_I64, _I64, _P, _I64, _P]),
    "nvfp4_hbm_stream_chunk_bytes": (_I64, []),
    "nvfp4_hbm_stream_ceiling": (_INT, [_P, _I64, _P, _I64, _P]),
    "nvfp4_status_string": (ctypes.c_char_p, [_INT]),
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_build_info": (ctypes.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({detail})")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with "
                                  "`python nvfp4_block_scaled_swiglu_amd/build.py`")
            l = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(l, name)
                fn.restype = res
                fn.argtypes = args
            _lib = l
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != NVFP4_OK:
        detail = lib().nvfp4_last_error().decode(errors="replace")
        raise Nvfp4Error(rc, where, detail)


# ---- dispatch policy and counters --------------------------------------------------------
#
# Strict (the default): a failing call raises Nvfp4Error. Non-strict: the call returns
# None and counts a fallback. The library validates every argument before it enqueues
# anything, so after a failure every buffer the caller passed, in particular NVFP4
# bytes already produced, is as it was (the two-pass producer's workspace aside), and
# the caller can fall back through them without quantizing twice ("FC2 NVFP4
# Scheduling Results", "Production Integration": fallback through the produced bytes,
# strict mode on request, dispatch and fallback counts per block). Nothing here
# computes a result itself. NVFP4_STRICT=0 in the environment starts non-strict;
# set_strict() changes the default, and each entry point takes strict= per call.
STRICT = os.environ.get("NVFP4_STRICT", "1") != "0"

# per entry point: attempts, successes, fallbacks (non-strict failures) and failures
# (strict failures, raised)
COUNTERS: Dict[str, Dict[str, int]] = {}
# the status and detail of the most recent fallback per entry point
LAST_FALLBACK: Dict[str, Tuple[int, str]] = {}


def set_strict(flag: bool) -> None:
    global STRICT
    STRICT = bool(flag)


def dispatch_counters() -> Dict[str, Dict[str, int]]:
    """A copy of the per-entry-point counters."""
    return {k: dict(v) for k, v in COUNTERS.items()}


def _call(name: str, *args, strict: Optional[bool] = None) -> bool:
    """Call entry point `name`; True on success. On failure raise (strict) or count a
    fallback and return False (non-strict)."""
    rc = getattr(lib(), name)(*args)
    c = COUNTERS.setdefault(name, {"attempts": 0, "successes": 0, "fallbacks": 0, "failures": 0})
    c["attempts"] += 1
    if rc == NVFP4_OK:
        c["successes"] += 1
        return True
    if STRICT if strict is None else strict:
        c["failures"] += 1
        _check(rc, name)
    c["fallbacks"] += 1
    LAST_FALLBACK[name] = (rc, lib().nvfp4_last_error().decode(errors="replace"))
    return False


# ---- sizes ---------------------------------------------------------------------------------

def nvfp4_padded_rows(rows: int) -> int:
    return int(lib().nvfp4_padded_rows(rows))


def nvfp4_scale_rows(rows: int) -> int:
    return int(lib().nvfp4_scale_rows(rows))


def nvfp4_scale_cols(k: int) -> int:
    return int(lib().nvfp4_scale_cols(k))


def nvfp4_qdata_bytes(rows: int, k: int) -> int:
    return int(lib().nvfp4_qdata_bytes(rows, k))


def nvfp4_scale_bytes(rows: int, k: int) -> int:
    return int(lib().nvfp4_scale_bytes(rows, k))


def nvfp4_quantize_workspace_bytes() -> int:
    return int(lib().nvfp4_quantize_workspace_bytes())


def nvfp4_status_string(status: int) -> str:
    return lib().nvfp4_status_string(status).decode()


def nvfp4_build_info() -> str:
    return lib().nvfp4_build_info().decode()


def nvfp4_init() -> None:
    _check(lib().nvfp4_init(), "nvfp4_init")


# ---- tensors -------------------------------------------------------------------------------

@dataclass
class Nvfp4Tensor:
    """A quantized [rows, k] tensor as the library lays it out in device memory."""
    qdata: "torch.Tensor"         # uint8 [padded_rows, k/2]
    scales: "torch.Tensor"        # uint8 [scale_rows * scale_cols], 128x4-tiled
    global_scale: "torch.Tensor"  # float32 [1]
    rows: int                     # logical rows
    k: int

    @property
    def padded_rows(self) -> int:
        return nvfp4_padded_rows(self.rows)


def empty_nvfp4(rows: int, k: int, device) -> Optional[Nvfp4Tensor]:
    import torch
    return Nvfp4Tensor(
        qdata=torch.empty((nvfp4_padded_rows(rows), k // 2), dtype=torch.uint8, device=device),
        scales=torch.empty((nvfp4_scale_bytes(rows, k),), dtype=torch.uint8, device=device),
        global_scale=torch.empty((1,), dtype=torch.float32, device=device),
        rows=rows, k=k)


_workspaces: Dict[Tuple[int, int], "torch.Tensor"] = {}


def _workspace(device, stream_handle: int):
    """A producer workspace per (device, stream), so that calls on different streams
    never share one. It starts zero-filled, as the library requires; every completed
    call leaves it zero-filled again."""
    import torch
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_handle)
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.zeros((nvfp4_quantize_workspace_bytes(),), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _stream_handle(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _bf16_2d(t, name: str):
    import torch
    if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_cuda:
        raise ValueError(f"{name} must be a 2-D bfloat16 CUDA tensor")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t


def nvfp4_quantize_swiglu(gate, up, out: Optional[Nvfp4Tensor] = None, m: Optional[int] = None,
                          workspace=None, stream=None, strict: Optional[bool] = None) -> Optional[Nvfp4Tensor]:
    """Fused y = RN_bf16(silu_bf16(gate) * up) -> NVFP4 (QDATA, 128x4-tiled scales, global scale)."""
    _bf16_2d(gate, "gate")
    _bf16_2d(up, "up")
    m = gate.shape[0] if m is None else m
    k = gate.shape[1]
    if up.shape[1] != k or up.shape[0] < m or gate.shape[0] < m:
        raise ValueError("gate/up shapes disagree")
    out = empty_nvfp4(m, k, gate.device) if out is None else out
    sh = _stream_handle(stream)
    ws = _workspace(gate.device, sh) if workspace is None else workspace
    if not _call("nvfp4_quantize_swiglu", gate.data_ptr(), gate.stride(0), up.data_ptr(), up.stride(0), m, k,
                 out.qdata.data_ptr(), out.scales.data_ptr(), out.global_scale.data_ptr(), ws.data_ptr(), sh,
                 strict=strict):
        return None
    return out


def nvfp4_quantize_swiglu_noalloc(gate, up, out: Nvfp4Tensor, m: Optional[int] = None, stream=None,
                                  strict: Optional[bool] = None) -> Optional[Nvfp4Tensor]:
    """nvfp4_quantize_swiglu with the library's fixed device scratch instead of a
    workspace, into the caller's preallocated `out` (nothing is allocated here or in
    the library; nvfp4_init must have run on the device). Calls overlapping on one GPU
    race on the shared scratch."""
    _bf16_2d(gate, "gate")
    _bf16_2d(up, "up")
    m = gate.shape[0] if m is None else m
    k = gate.shape[1]
    if up.shape[1] != k or up.shape[0] < m or gate.shape[0] < m:
        raise ValueError("gate/up shapes disagree")
    if out.rows != m or out.k != k:
        raise ValueError("out must be an Nvfp4Tensor for the same rows and k")
    if not _call("nvfp4_quantize_swiglu_noalloc", gate.data_ptr(), gate.stride(0), up.data_ptr(), up.stride(0), m,
                 k, out.qdata.data_ptr(), out.scales.data_ptr(), out.global_scale.data_ptr(),
                 _stream_handle(stream), strict=strict):
        return None
    return out


def nvfp4_quantize(x, out: Optional[Nvfp4Tensor] = None, rows: Optional[int] = None, workspace=None,
                   stream=None, strict: Optional[bool] = None) -> Optional[Nvfp4Tensor]:
    """Plain NVFP4 quantization of a bf16 [rows, k] tensor (y = x)."""
    _bf16_2d(x, "x")
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1]
    out = empty_nvfp4(rows, k, x.device) if out is None else out
    sh = _stream_handle(stream)
    ws = _workspace(x.device, sh) if workspace is None else workspace
    if not _call("nvfp4_quantize", x.data_ptr(), x.stride(0), rows, k, out.qdata.data_ptr(), out.scales.data_ptr(),
                 out.global_scale.data_ptr(), ws.data_ptr(), sh,
                 strict=strict):
        return None
    return out


def nvfp4_quantize_modulate(x, scale, shift, out: Optional[Nvfp4Tensor] = None, rows: Optional[int] = None,
                            workspace=None, stream=None, strict: Optional[bool] = None) -> Optional[Nvfp4Tensor]:
    """NVFP4 of y = RN_bf16(fma_fp32(x, 1 + scale, shift)) (scale, shift: bf16 [k])."""
    import torch
    _bf16_2d(x, "x")
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1]
    for name, t in (("scale", scale), ("shift", shift)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (k,) or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor of shape ({k},)")
    out = empty_nvfp4(rows, k, x.device) if out is None else out
    sh = _stream_handle(stream)
    ws = _workspace(x.device, sh) if workspace is None else workspace
    if not _call("nvfp4_quantize_modulate", x.data_ptr(), x.stride(0), rows, k, scale.data_ptr(), shift.data_ptr(),
                 out.qdata.data_ptr(), out.scales.data_ptr(), out.global_scale.data_ptr(), ws.data_ptr(), sh,
                 strict=strict):
        return None
    return out


def _amax_ptr(amax) -> int:
    import torch
    if not isinstance(amax, torch.Tensor) or amax.dtype != torch.float32 or not amax.is_cuda or amax.numel() < 1:
        raise ValueError("amax must be a float32 CUDA tensor holding at least one element")
    return amax.data_ptr()


def nvfp4_quantize_swiglu_amax(gate, up, amax, out: Optional[Nvfp4Tensor] = None, m: Optional[int] = None,
                               stream=None, strict: Optional[bool] = None) -> Optional[Nvfp4Tensor]:
    """Single-read SwiGLU -> NVFP4 with the caller's tensor amax (a device float32 scalar)."""
    _bf16_2d(gate, "gate")
    _bf16_2d(up, "up")
    m = gate.shape[0] if m is None else m
    k = gate.shape[1]
    if up.shape[1] != k or up.shape[0] < m or gate.shape[0] < m:
        raise ValueError("gate/up shapes disagree")
    out = empty_nvfp4(m, k, gate.device) if out is None else out
    if not _call("nvfp4_quantize_swiglu_amax", gate.data_ptr(), gate.stride(0), up.data_ptr(), up.stride(0), m, k,
                 _amax_ptr(amax), out.qdata.data_ptr(), out.scales.data_ptr(), out.global_scale.data_ptr(),
                 _stream_handle(stream), strict=strict):
        return None
    return out


def nvfp4_quantize_amax(x, amax, out: Optional[Nvfp4Tensor] = None, rows: Optional[int] = None,
                        stream=None, strict: Optional[bool] = None) -> Optional[Nvfp4Tensor]:
    """Single-read plain NVFP4 quantization with the caller's tensor amax."""
    _bf16_2d(x, "x")
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1]
    out = empty_nvfp4(rows, k, x.device) if out is None else out
    if not _call("nvfp4_quantize_amax", x.data_ptr(), x.stride(0), rows, k, _amax_ptr(amax), out.qdata.data_ptr(),
                 out.scales.data_ptr(), out.global_scale.data_ptr(), _stream_handle(stream), strict=strict):
        return None
    return out


def nvfp4_gemm_bf16out(a: Nvfp4Tensor, w: Nvfp4Tensor, out=None, stream=None, strict: Optional[bool] = None):
    """D[m_padded, n] = RN_bf16(g_a g_w sum_k deq(A) deq(W)), FP32 accumulation."""
    import torch
    if a.k != w.k:
        raise ValueError("k mismatch")
    m_pad = a.padded_rows
    n = w.rows
    if out is None:
        out = torch.empty((m_pad, n), dtype=torch.bfloat16, device=a.qdata.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (m_pad, n) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [m_padded, n] tensor")
    if not _call("nvfp4_gemm_bf16out", a.qdata.data_ptr(), a.scales.data_ptr(), a.global_scale.data_ptr(),
                 w.qdata.data_ptr(), w.scales.data_ptr(), w.global_scale.data_ptr(), out.data_ptr(), m_pad, n, a.k,
                 _stream_handle(stream), strict=strict):
        return None
    return out


def nvfp4_gemm_bf16out_fused(a: Nvfp4Tensor, w: Nvfp4Tensor, bias=None, gate=None, residual=None, out=None,
                             stream=None, strict: Optional[bool] = None):
    """D = RN_bf16(residual + gate * RN_bf16(g_a g_w sum + bias)) (each term optional;
    without a residual D is the biased GEMM output). out may be residual (in place)."""
    import torch
    if a.k != w.k:
        raise ValueError("k mismatch")
    m_pad = a.padded_rows
    n = w.rows
    if out is None:
        out = torch.empty((m_pad, n), dtype=torch.bfloat16, device=a.qdata.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (m_pad, n) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [m_padded, n] tensor")
    for name, t, shape in (("bias", bias, (n,)), ("gate", gate, (n,)), ("residual", residual, (m_pad, n))):
        if t is not None and (t.dtype != torch.bfloat16 or tuple(t.shape) != shape or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor of shape {shape}")
    ptr = lambda t: None if t is None else t.data_ptr()
    if not _call("nvfp4_gemm_bf16out_fused", a.qdata.data_ptr(), a.scales.data_ptr(), a.global_scale.data_ptr(),
                 w.qdata.data_ptr(), w.scales.data_ptr(), w.global_scale.data_ptr(), out.data_ptr(), m_pad, n, a.k,
                 ptr(bias), ptr(gate), ptr(residual), _stream_handle(stream), strict=strict):
        return None
    return out


def interleave_swiglu_weight(w_gate, w_up):
    """[n_half, k] gate and up weights -> [2 n_half, k] with rows interleaved in chunks
    of 8 (the layout nvfp4_gemm_swiglu_pair expects)."""
    n_half, k = w_gate.shape
    if tuple(w_up.shape) != (n_half, k) or n_half % 8 != 0:
        raise ValueError("gate and up weights must be [n_half, k] with n_half % 8 == 0")
    return _torch_stack_chunks(w_gate, w_up)


def _torch_stack_chunks(a, b):
    import torch
    n_half, k = a.shape
    return torch.stack([a.reshape(n_half // 8, 8, k), b.reshape(n_half // 8, 8, k)], dim=1).reshape(2 * n_half, k)


def nvfp4_gemm_swiglu_pair(a: Nvfp4Tensor, w: Nvfp4Tensor, bias=None, amax=None, amax_rows: Optional[int] = None,
                           gate_out=None, up_out=None, stream=None, strict: Optional[bool] = None):
    """FC1 with the SwiGLU pair epilogue: returns (gate, up) bf16 [m_padded, n_half];
    if amax (a float32 CUDA tensor, set by the caller) is given, max |silu(gate) * up|
    over the logical rows is folded into it."""
    import torch
    if a.k != w.k or w.rows % 16 != 0:
        raise ValueError("k mismatch or weight rows not a multiple of 16")
    m_pad = a.padded_rows
    n_half = w.rows // 2
    dev = a.qdata.device
    gate_out = torch.empty((m_pad, n_half), dtype=torch.bfloat16, device=dev) if gate_out is None else gate_out
    up_out = torch.empty((m_pad, n_half), dtype=torch.bfloat16, device=dev) if up_out is None else up_out
    for name, t in (("gate_out", gate_out), ("up_out", up_out)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (m_pad, n_half) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 [m_padded, n_half] tensor")
    if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (2 * n_half,)):
        raise ValueError("bias must be bfloat16 [2 n_half] (interleaved order)")
    if not _call("nvfp4_gemm_swiglu_pair", a.qdata.data_ptr(), a.scales.data_ptr(), a.global_scale.data_ptr(),
                 w.qdata.data_ptr(), w.scales.data_ptr(), w.global_scale.data_ptr(), gate_out.data_ptr(),
                 up_out.data_ptr(), m_pad, n_half, a.k, None if bias is None else bias.data_ptr(),
                 None if amax is None else _amax_ptr(amax), a.rows if amax_rows is None else amax_rows,
                 _stream_handle(stream), strict=strict):
        return None
    return gate_out, up_out


def nvfp4_gemm_bf16out_clock(a: Nvfp4Tensor, w: Nvfp4Tensor, out, clk, stream=None):
    """nvfp4_gemm_bf16out into `out` with per-workgroup shader-clock stamps in `clk`
    (an int64 CUDA tensor [slots, 2]: cycles, 100 MHz ticks); a measurement aid."""
    import torch
    m_pad, n = a.padded_rows, w.rows
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (m_pad, n) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [m_padded, n] tensor")
    if clk.dtype != torch.int64 or clk.dim() != 2 or clk.shape[1] != 2 or not clk.is_contiguous():
        raise ValueError("clk must be a contiguous int64 [slots, 2] tensor")
    _call("nvfp4_gemm_bf16out_clock", a.qdata.data_ptr(), a.scales.data_ptr(), a.global_scale.data_ptr(),
          w.qdata.data_ptr(), w.scales.data_ptr(), w.global_scale.data_ptr(), out.data_ptr(), m_pad, n, a.k,
          clk.data_ptr(), clk.shape[0], _stream_handle(stream))
    return out


def nvfp4_mfma_ceiling(workgroups: int, iters: int, stream=None):
    """Run the matrix-core ceiling kernel once (a measurement aid, not a step of the
    method). Returns the per-wave uint64 tensor [workgroups * 4, 2] of (shader-clock
    cycles, 100 MHz ticks); time the call with events for the rate. Each wave issues
    iters * 4 MFMAs of 2 * 32 * 32 * 16 FLOP."""
    import torch
    nbytes = lib().nvfp4_mfma_ceiling_out_bytes(workgroups)
    out = torch.zeros((max(nbytes, 16) // 8,), dtype=torch.int64, device=torch.cuda.current_device())
    _call("nvfp4_mfma_ceiling", workgroups, iters, out.data_ptr(), nbytes, _stream_handle(stream))
    return out.view(-1, 2)


def nvfp4_hbm_stream_ceiling(src, read_bytes: int, dst, write_bytes: int, stream=None) -> int:
    """Run the HBM streaming probe once (a measurement aid, not a step of the method):
    read read_bytes of the CUDA tensor src, write about write_bytes of dst. Returns the
    bytes actually written; time the call with events for the rate."""
    chunk = int(lib().nvfp4_hbm_stream_chunk_bytes())
    if src.numel() * src.element_size() < read_bytes or dst.numel() * dst.element_size() < max(write_bytes, 16):
        raise ValueError("src or dst smaller than the requested bytes")
    _call("nvfp4_hbm_stream_ceiling", src.data_ptr(), read_bytes, dst.data_ptr(), write_bytes,
          _stream_handle(stream))
    chunks = read_bytes // chunk
    return 16 * chunks * (write_bytes // (16 * chunks))


def nvfp4_silu_bf16(x, out=None, stream=None):
    """The producer's correctly rounded bf16 silu applied elementwise (uint16/int16/bf16 bits)."""
    import torch
    out = torch.empty_like(x) if out is None else out
    _call("nvfp4_silu_bf16", x.data_ptr(), out.data_ptr(), x.numel(), _stream_handle(stream))
    return out
