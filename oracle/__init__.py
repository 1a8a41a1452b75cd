"""CPU oracle of the NVFP4 SwiGLU producer and block-scaled GEMM (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP library. The arithmetic, its readings of the pages and its pins
are described at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# NVFP4_ORACLE_LIB lets a pin-strength check load a deliberately altered build.
_LIB_PATH = os.environ.get("NVFP4_ORACLE_LIB", os.path.join(HERE, "liboracle.so"))
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "oracle_rn_bf16": (ctypes.c_uint16, [ctypes.c_double]),
        "oracle_silu_bf16": (ctypes.c_uint16, [ctypes.c_uint16]),
        "oracle_silu_table": (None, [_P]),
        "oracle_swiglu_bf16": (ctypes.c_uint16, [ctypes.c_uint16, ctypes.c_uint16, _P]),
        "oracle_ue4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
        "oracle_e2m1_value": (ctypes.c_double, [ctypes.c_uint8]),
        "oracle_global_scale": (ctypes.c_float, [ctypes.c_double]),
        "oracle_block_scale": (ctypes.c_uint8, [ctypes.c_double, ctypes.c_float]),
        "oracle_e2m1_code": (ctypes.c_uint8, [ctypes.c_double, ctypes.c_uint8, ctypes.c_float]),
        "oracle_padded_rows": (_I64, [_I64]),
        "oracle_scale_rows": (_I64, [_I64]),
        "oracle_scale_cols": (_I64, [_I64]),
        "oracle_scale_offset": (_I64, [_I64, _I64, _I64]),
        "oracle_quantize": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _I64, _P, _P, _P, _P,
                                           ctypes.c_int]),
        "oracle_quantize_amax": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _I64, ctypes.c_double, _P, _P,
                                                _P, ctypes.c_int]),
        "oracle_modulate_bf16": (ctypes.c_uint16, [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_uint16]),
        "oracle_quantize_modulate": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, ctypes.c_int]),
        "oracle_gemm_swiglu_rows": (ctypes.c_int, [_P, _P, _I64, ctypes.c_float, _P, _P, _I64, ctypes.c_float,
                                                   _I64, _P, _I64, _P, _P, _P, _P, ctypes.c_int]),
        "oracle_gemm_rows_ex": (ctypes.c_int, [_P, _P, _I64, ctypes.c_float, _P, _P, _I64, ctypes.c_float,
                                               _I64, _P, _I64, _P, _P, _P, _I64, _P, _P, ctypes.c_int]),
        "oracle_gemm_rows": (ctypes.c_int, [_P, _P, _I64, ctypes.c_float, _P, _P, _I64,
                                            ctypes.c_float, _I64, _P, _I64, _P, ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---- scalar steps (used by the pins) ----------------------------------------------

def rn_bf16(v: float) -> int:
    return int(_load().oracle_rn_bf16(float(v)))


def silu_bf16(x_bits: int) -> int:
    return int(_load().oracle_silu_bf16(x_bits))


def silu_table() -> np.ndarray:
    tab = np.empty(65536, dtype=np.uint16)
    _load().oracle_silu_table(tab.ctypes.data)
    return tab


def swiglu_bf16(gate_bits: int, up_bits: int) -> int:
    return int(_load().oracle_swiglu_bf16(gate_bits, up_bits, None))


def ue4m3_value(b: int) -> float:
    return float(_load().oracle_ue4m3_value(b))


def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(code))


def global_scale(amax: float) -> float:
    return float(_load().oracle_global_scale(amax))


def block_scale(bmax: float, g: float) -> int:
    return int(_load().oracle_block_scale(bmax, g))


def e2m1_code(y: float, s: int, g: float) -> int:
    return int(_load().oracle_e2m1_code(y, s, g))


def padded_rows(rows: int) -> int:
    return int(_load().oracle_padded_rows(rows))


def scale_rows(rows: int) -> int:
    return int(_load().oracle_scale_rows(rows))


def scale_cols(k: int) -> int:
    return int(_load().oracle_scale_cols(k))


def scale_offset(r: int, c: int, cpad: int) -> int:
    return int(_load().oracle_scale_offset(r, c, cpad))


def qdata_bytes(rows: int, k: int) -> int:
    return padded_rows(rows) * k // 2


def scale_bytes(rows: int, k: int) -> int:
    return scale_rows(rows) * scale_cols(k)


# ---- whole tensors ---------------------------------------------------------------

def quantize(x: np.ndarray, up: Optional[np.ndarray] = None, m: Optional[int] = None,
             return_y: bool = False, threads: Optional[int] = None):
    """Quantize y = swiglu(x, up) (up given) or y = x of shape [m, k] (bf16 bits, uint16).

    Returns (qdata [m_pad, k/2] uint8, scales [scale_bytes] uint8, g float[, y]).
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m = x.shape[0] if m is None else m
    k = x.shape[1]
    if up is not None:
        up = np.ascontiguousarray(up, dtype=np.uint16)
        assert up.shape[1] == k and up.shape[0] >= m
    qdata = np.empty((padded_rows(m), k // 2), dtype=np.uint8)
    scales = np.empty(scale_bytes(m, k), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    y = np.empty((m, k), dtype=np.uint16) if return_y else None
    rc = _load().oracle_quantize(x.ctypes.data, k, None if up is None else up.ctypes.data, k, m, k,
                                 qdata.ctypes.data, scales.ctypes.data, g.ctypes.data,
                                 None if y is None else y.ctypes.data,
                                 threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_quantize failed ({rc})")
    if return_y:
        return qdata, scales, float(g[0]), y
    return qdata, scales, float(g[0])


def quantize_amax(x: np.ndarray, up: Optional[np.ndarray], amax: float, m: Optional[int] = None,
                  threads: Optional[int] = None):
    """O11: quantize y = swiglu(x, up) (up given) or y = x with the caller's amax
    instead of max |y|. Returns (qdata, scales, g) as ``quantize``."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m = x.shape[0] if m is None else m
    k = x.shape[1]
    if up is not None:
        up = np.ascontiguousarray(up, dtype=np.uint16)
        assert up.shape[1] == k and up.shape[0] >= m
    qdata = np.empty((padded_rows(m), k // 2), dtype=np.uint8)
    scales = np.empty(scale_bytes(m, k), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    rc = _load().oracle_quantize_amax(x.ctypes.data, k, None if up is None else up.ctypes.data, k, m, k,
                                      float(amax), qdata.ctypes.data, scales.ctypes.data, g.ctypes.data,
                                      threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_quantize_amax failed ({rc})")
    return qdata, scales, float(g[0])


def modulate_bf16(x: int, scale: int, shift: int) -> int:
    return int(_load().oracle_modulate_bf16(x, scale, shift))


def quantize_modulate(x: np.ndarray, scale: np.ndarray, shift: np.ndarray, m: Optional[int] = None,
                      return_y: bool = False, threads: Optional[int] = None):
    """O13 + O3-O8: plain NVFP4 quantization of y = RN_bf16(fma_fp32(x, 1 + scale, shift))
    (bf16 bits; scale, shift [k]). Returns (qdata, scales, g[, y])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m = x.shape[0] if m is None else m
    k = x.shape[1]
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    shift = np.ascontiguousarray(shift, dtype=np.uint16)
    assert scale.shape == (k,) and shift.shape == (k,)
    qdata = np.empty((padded_rows(m), k // 2), dtype=np.uint8)
    scales = np.empty(scale_bytes(m, k), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    y = np.empty((m, k), dtype=np.uint16) if return_y else None
    rc = _load().oracle_quantize_modulate(x.ctypes.data, k, m, k, scale.ctypes.data, shift.ctypes.data,
                                          qdata.ctypes.data, scales.ctypes.data, g.ctypes.data,
                                          None if y is None else y.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_quantize_modulate failed ({rc})")
    if return_y:
        return qdata, scales, float(g[0]), y
    return qdata, scales, float(g[0])


def gemm_rows(a_q: np.ndarray, a_s: np.ndarray, a_rows: int, ga: float, w_q: np.ndarray,
              w_s: np.ndarray, n: int, gw: float, k: int, rows: Sequence[int],
              threads: Optional[int] = None) -> np.ndarray:
    """Exact RN_bf16 GEMM output for the selected activation rows: [len(rows), n] bf16 bits."""
    a_q = np.ascontiguousarray(a_q, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.uint8)
    w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
    w_s = np.ascontiguousarray(w_s, dtype=np.uint8)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((rows.shape[0], n), dtype=np.uint16)
    rc = _load().oracle_gemm_rows(a_q.ctypes.data, a_s.ctypes.data, a_rows, ga, w_q.ctypes.data,
                                  w_s.ctypes.data, n, gw, k, rows.ctypes.data, rows.shape[0],
                                  out.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm_rows failed ({rc})")
    return out


def gemm_rows_ex(a_q: np.ndarray, a_s: np.ndarray, a_rows: int, ga: float, w_q: np.ndarray,
                 w_s: np.ndarray, n: int, gw: float, k: int, rows: Sequence[int],
                 bias: Optional[np.ndarray] = None, gate: Optional[np.ndarray] = None,
                 res: Optional[np.ndarray] = None, threads: Optional[int] = None):
    """O12: (D1, D) for the selected activation rows, [len(rows), n] bf16 bits each.
    bias, gate: bf16 bits [n] or None; res: bf16 bits [a_padded_rows, >= n] or None
    (indexed by activation row). D = D1 without a residual."""
    a_q = np.ascontiguousarray(a_q, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.uint8)
    w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
    w_s = np.ascontiguousarray(w_s, dtype=np.uint8)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    gate = None if gate is None else np.ascontiguousarray(gate, dtype=np.uint16)
    res = None if res is None else np.ascontiguousarray(res, dtype=np.uint16)
    if bias is not None:
        assert bias.shape == (n,)
    if gate is not None:
        assert gate.shape == (n,)
    d1 = np.empty((rows.shape[0], n), dtype=np.uint16)
    d = np.empty((rows.shape[0], n), dtype=np.uint16)
    rc = _load().oracle_gemm_rows_ex(a_q.ctypes.data, a_s.ctypes.data, a_rows, ga, w_q.ctypes.data,
                                     w_s.ctypes.data, n, gw, k, rows.ctypes.data, rows.shape[0],
                                     None if bias is None else bias.ctypes.data,
                                     None if gate is None else gate.ctypes.data,
                                     None if res is None else res.ctypes.data,
                                     0 if res is None else res.shape[1], d1.ctypes.data, d.ctypes.data,
                                     threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm_rows_ex failed ({rc})")
    return d1, d


def gemm_swiglu_rows(a_q: np.ndarray, a_s: np.ndarray, a_rows: int, ga: float, w_q: np.ndarray,
                     w_s: np.ndarray, n_half: int, gw: float, k: int, rows: Sequence[int],
                     bias: Optional[np.ndarray] = None, threads: Optional[int] = None):
    """O14: (gate, up, ymax) for the selected activation rows: gate and up are bf16 bits
    [len(rows), n_half], ymax float32 [len(rows)] (max |RN_bf16(silu(gate) * up)|).
    The weight holds 2 n_half rows, gate and up interleaved in chunks of 8."""
    a_q = np.ascontiguousarray(a_q, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.uint8)
    w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
    w_s = np.ascontiguousarray(w_s, dtype=np.uint8)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    if bias is not None:
        assert bias.shape == (2 * n_half,)
    gate = np.empty((rows.shape[0], n_half), dtype=np.uint16)
    up = np.empty((rows.shape[0], n_half), dtype=np.uint16)
    ymax = np.empty(rows.shape[0], dtype=np.float32)
    rc = _load().oracle_gemm_swiglu_rows(a_q.ctypes.data, a_s.ctypes.data, a_rows, ga, w_q.ctypes.data,
                                         w_s.ctypes.data, n_half, gw, k, rows.ctypes.data, rows.shape[0],
                                         None if bias is None else bias.ctypes.data, gate.ctypes.data,
                                         up.ctypes.data, ymax.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm_swiglu_rows failed ({rc})")
    return gate, up, ymax


def interleave_swiglu_rows(gate_w: np.ndarray, up_w: np.ndarray) -> np.ndarray:
    """The chunk-of-8 interleaving of O14: [n_half, k] gate and up rows -> [2 n_half, k]."""
    n_half, k = gate_w.shape
    assert up_w.shape == (n_half, k) and n_half % 8 == 0
    out = np.empty((2 * n_half, k), dtype=gate_w.dtype)
    v = out.reshape(n_half // 8, 2, 8, k)
    v[:, 0] = gate_w.reshape(n_half // 8, 8, k)
    v[:, 1] = up_w.reshape(n_half // 8, 8, k)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
