"""Seeded synthetic inputs for the NVFP4 SwiGLU -> FC2 path.

This package draws numbers and describes workloads; it holds none of the
quantization or GEMM arithmetic. The HIP path and the CPU oracle are both fed
the bytes it produces. The generator itself is defined in ``synth.c``.

Workloads follow the shapes of the FC2 projection of one 1344x768, 124-frame
video (37,810 packed tokens, hidden 5,376, MLP width 14,336) from the pages'
production profile ("gb10-post-fc2-production-profile" summary, ``workload``
key) and the FC2 scheduling results page ("Canonical Operation").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libsynth.so")
_lib = None

# Tensor tags: each tensor of a workload draws from its own stream.
TAG_GATE = 1
TAG_UP = 2
TAG_WEIGHT = 3
TAG_OUTLIER = 5
TAG_PLAIN_X = {"qkv": 11, "attn_out": 21, "fc1": 31}
TAG_PLAIN_W = {"qkv": 12, "attn_out": 22, "fc1": 32, "qkv_pages": 42}


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
    lib.synth_draw.restype = ctypes.c_uint64
    lib.synth_draw.argtypes = [ctypes.c_uint64] * 3
    lib.synth_normal.restype = ctypes.c_double
    lib.synth_normal.argtypes = [ctypes.c_uint64] * 3
    lib.synth_outlier_mask.restype = ctypes.c_int
    lib.synth_outlier_mask.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                       ctypes.c_uint64, ctypes.c_int64]
    lib.synth_normal_bf16.restype = ctypes.c_int
    lib.synth_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                      ctypes.c_float, ctypes.c_void_p, ctypes.c_int]
    lib.synth_bytes.restype = ctypes.c_int
    lib.synth_bytes.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int]
    _lib = lib
    return lib


def draw(seed: int, tag: int, i: int) -> int:
    return int(_load().synth_draw(seed, tag, i))


def normal(seed: int, tag: int, i: int) -> float:
    return float(_load().synth_normal(seed, tag, i))


def outlier_mask(cols: int, seed: int, n_out: int, tag: int = TAG_OUTLIER) -> np.ndarray:
    mask = np.zeros(cols, dtype=np.uint8)
    rc = _load().synth_outlier_mask(mask.ctypes.data, cols, seed, tag, n_out)
    if rc != 0:
        raise ValueError(f"synth_outlier_mask failed ({rc})")
    return mask


def normal_bf16(rows: int, cols: int, seed: int, tag: int, sigma: float,
                mask: Optional[np.ndarray] = None, ld: Optional[int] = None,
                threads: Optional[int] = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of shape [rows, ld]; columns >= cols are zero."""
    ld = cols if ld is None else ld
    out = np.zeros((rows, ld), dtype=np.uint16) if ld != cols else np.empty((rows, ld), dtype=np.uint16)
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.uint8)
        assert mask.shape == (cols,)
    rc = _load().synth_normal_bf16(out.ctypes.data, rows, cols, ld, seed, tag, sigma,
                                   None if mask is None else mask.ctypes.data,
                                   threads or default_threads())
    if rc != 0:
        raise ValueError(f"synth_normal_bf16 failed ({rc})")
    return out


def uniform_bytes(n: int, seed: int, tag: int, lo: int = 0, hi: int = 255,
                  threads: Optional[int] = None) -> np.ndarray:
    """n seeded uniform bytes in [lo, hi]."""
    out = np.empty(n, dtype=np.uint8)
    rc = _load().synth_bytes(out.ctypes.data, n, seed, tag, lo, hi, threads or default_threads())
    if rc != 0:
        raise ValueError(f"synth_bytes failed ({rc})")
    return out


def padded_rows(m: int) -> int:
    """Rows after the producer's padding: the next multiple of 16."""
    return (m + 15) // 16 * 16


@dataclass
class Workload:
    """One GEMM workload: activation [m, k] (SwiGLU pair or plain x), weight [n, k]."""
    name: str
    m: int
    n: int
    k: int
    seed: int
    swiglu: bool                 # True: gate/up pair through SwiGLU; False: plain x
    outliers: bool = False       # 1% of channels scaled x20
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    tag_x: int = TAG_PLAIN_X["qkv"]
    tag_w: int = TAG_WEIGHT
    meta: Dict[str, str] = field(default_factory=dict)

    @property
    def m_pad(self) -> int:
        return padded_rows(self.m)

    @property
    def n_outliers(self) -> int:
        return int(round(0.01 * self.k)) if self.outliers else 0

    def mask(self) -> Optional[np.ndarray]:
        if not self.outliers:
            return None
        return outlier_mask(self.k, self.seed, self.n_outliers)

    def activations(self, rows: Optional[int] = None, threads: Optional[int] = None):
        """SwiGLU: (gate, up); plain: (x,). rows < m generates the leading rows only
        (the generator is counter-based, so a prefix is identical to the full tensor's)."""
        rows = self.m if rows is None else rows
        mask = self.mask()
        if self.swiglu:
            gate = normal_bf16(rows, self.k, self.seed, TAG_GATE, self.x_sigma, mask, threads=threads)
            up = normal_bf16(rows, self.k, self.seed, TAG_UP, self.x_sigma, mask, threads=threads)
            return gate, up
        return (normal_bf16(rows, self.k, self.seed, self.tag_x, self.x_sigma, mask, threads=threads),)

    def weight(self, threads: Optional[int] = None) -> np.ndarray:
        return normal_bf16(self.n, self.k, self.seed, self.tag_w, self.w_sigma, None, threads=threads)

    @property
    def gemm_flops(self) -> float:
        """Dense FLOPs counted on the logical M, as the pages do for FC2."""
        return 2.0 * self.m * self.n * self.k


TINY = Workload("tiny", m=256, n=512, k=1024, seed=0, swiglu=True)
MID = Workload("mid_fc2_slice", m=4096, n=5376, k=14336, seed=1, swiglu=True, outliers=True)
FC2 = Workload("fc2_canonical", m=37810, n=5376, k=14336, seed=440420, swiglu=True, outliers=True)
QKV = Workload("qkv", m=37810, n=16128, k=5376, seed=7, swiglu=False,
               tag_x=TAG_PLAIN_X["qkv"], tag_w=TAG_PLAIN_W["qkv"])
ATTN_OUT = Workload("attn_out", m=37810, n=5376, k=7168, seed=7, swiglu=False,
                    tag_x=TAG_PLAIN_X["attn_out"], tag_w=TAG_PLAIN_W["attn_out"])
FC1 = Workload("fc1", m=37810, n=28672, k=5376, seed=7, swiglu=False,
               tag_x=TAG_PLAIN_X["fc1"], tag_w=TAG_PLAIN_W["fc1"])
# The QKV projection at the width the pages' kernel grid implies (168 N-tiles of 128:
# 21,504 = 3 x 7,168), beside the configured 16,128.
QKV_PAGES = Workload("qkv_pages", m=37810, n=21504, k=5376, seed=7, swiglu=False,
                     tag_x=TAG_PLAIN_X["qkv"], tag_w=TAG_PLAIN_W["qkv_pages"])
RAGGED_M: List[int] = [37711, 37725, 37742, 37774, 37809, 37838, 37966, 38222]
RAGGED = [Workload(f"fc2_ragged_m{m}", m=m, n=5376, k=14336, seed=100 + i, swiglu=True, outliers=True)
          for i, m in enumerate(RAGGED_M)]
PLAIN = [QKV, ATTN_OUT, FC1, QKV_PAGES]
ALL = [TINY, MID, FC2] + PLAIN + RAGGED
BY_NAME = {w.name: w for w in ALL}
