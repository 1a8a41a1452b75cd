"""Shared helpers for the parity tests, the smoke check and the benchmark: moving
seeded inputs to the GPU, running the HIP path through the C ABI, and comparing
with the oracle.

GEMM tolerance (the oracle is exact and rounds once to bf16):
  * per element |D - D_ref| <= ulp_bf16(max(|D_ref|, tau)), tau = 2^-8 * max |D_ref|
    over the checked set: one bf16 ulp, with a floor near zero where an FP32
    accumulation of thousands of terms cannot promise a relative bound;
  * ||D - D_ref||_F / ||D_ref||_F <= 2e-3.
The fused epilogue's bounds follow from this one (see fused_compare).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

REL_FRO_TOL = 2e-3


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(mag: np.ndarray) -> np.ndarray:
    mag = np.asarray(mag, dtype=np.float64)
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))
    return np.ldexp(1.0, np.maximum(e - 1, -126) - 7)


def gemm_compare(got_bits: np.ndarray, ref_bits: np.ndarray) -> Dict[str, float]:
    got = bf16_bits_to_f64(got_bits)
    ref = bf16_bits_to_f64(ref_bits)
    assert np.isfinite(got).all(), "non-finite GEMM output"
    diff = np.abs(got - ref)
    amax = float(np.abs(ref).max()) if ref.size else 0.0
    tau = 2.0 ** -8 * amax
    tol = ulp_bf16(np.maximum(np.abs(ref), tau))
    strict_tol = ulp_bf16(np.abs(ref))
    nref = float(np.sqrt((ref ** 2).sum()))
    fro = float(np.sqrt((diff ** 2).sum()) / nref) if nref > 0 else float(np.sqrt((diff ** 2).sum()))
    return {
        "checked": int(ref.size),
        "violations": int((diff > tol).sum()),
        "differing": int((got_bits != ref_bits).sum()),
        "over_1ulp_no_floor": int((diff > strict_tol).sum()),
        "max_abs_diff": float(diff.max()) if diff.size else 0.0,
        "rel_fro": fro,
        "tau": tau,
    }


def assert_gemm_close(got_bits: np.ndarray, ref_bits: np.ndarray, what: str = "") -> Dict[str, float]:
    st = gemm_compare(got_bits, ref_bits)
    assert st["violations"] == 0 and st["rel_fro"] <= REL_FRO_TOL, f"{what} GEMM out of tolerance: {st}"
    return st


def fused_compare(d1_got: np.ndarray, d1_ref: np.ndarray, plain_ref: np.ndarray,
                  d_got: Optional[np.ndarray] = None, d_ref: Optional[np.ndarray] = None,
                  gate: Optional[np.ndarray] = None) -> Dict[str, float]:
    """Tolerance of the fused epilogue, derived from the GEMM bar:
      * D1 = RN_bf16(X + bias): |D1 - D1_ref| <= ulp_bf16(max(|D1_ref|, tau)) with
        tau = 2^-8 max |X_ref| (X_ref: the unbiased output, plain_ref), the FP32
        accumulation floor of the plain GEMM, independent of the bias magnitude;
      * D = RN_bf16(res + gate D1): a D1 error e1 moves the exact sum by |gate| e1,
        and each side rounds once, so |D - D_ref| <= |gate| tol1 + ulp_bf16(max(|D|, |D_ref|)).
    """
    g1 = bf16_bits_to_f64(d1_got)
    r1 = bf16_bits_to_f64(d1_ref)
    x = bf16_bits_to_f64(plain_ref)
    assert np.isfinite(g1).all(), "non-finite D1"
    tau = 2.0 ** -8 * (float(np.abs(x).max()) if x.size else 0.0)
    tol1 = ulp_bf16(np.maximum(np.abs(r1), tau))
    out = {"checked": int(r1.size), "d1_violations": int((np.abs(g1 - r1) > tol1).sum()),
           "d1_differing": int((d1_got != d1_ref).sum()), "tau": tau}
    if d_got is not None:
        gd = bf16_bits_to_f64(d_got)
        rd = bf16_bits_to_f64(d_ref)
        gv = np.ones(r1.shape[1]) if gate is None else bf16_bits_to_f64(gate)
        tol = np.abs(gv)[None, :] * tol1 + ulp_bf16(np.maximum(np.abs(gd), np.abs(rd)))
        out["d_violations"] = int((np.abs(gd - rd) > tol).sum())
        out["d_differing"] = int((d_got != d_ref).sum())
    return out


PARITY_ROWS = 4096  # seeded logical rows sampled per large configuration


def sample_rows(m: int, m_pad: int, count: int, seed: int) -> np.ndarray:
    """Rows whose GEMM outputs are compared: `count` seeded logical rows, plus the rows
    on both sides of every 256-row tile boundary (the GEMM's M tiles) and of every
    128-row boundary in the last 512 rows (its quarter-tile tail), the last 64 logical
    rows, row 0, and every padding row [m, m_pad)."""
    rng = np.random.default_rng(seed)
    base = rng.choice(m, size=min(count, m), replace=False)
    b256 = np.arange(256, m_pad, 256)
    b128 = np.arange(max(128, (m_pad - 512) // 128 * 128), m_pad, 128)
    edges = np.concatenate([b256 - 1, b256, b128 - 1, b128])
    tail = np.arange(max(0, m - 64), m)
    pad = np.arange(m, m_pad)
    rows = np.unique(np.concatenate([base, edges, tail, [0], pad])).astype(np.int64)
    return rows[(rows >= 0) & (rows < m_pad)]


def to_device_bf16(bits: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def tensor_bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def run_quantize(x_bits: np.ndarray, up_bits: Optional[np.ndarray], device, m: Optional[int] = None):
    """HIP producer on seeded inputs; returns (Nvfp4Tensor, qdata np, scales np, g float)."""
    import nvfp4_block_scaled_swiglu_amd as nv
    x = to_device_bf16(x_bits, device)
    if up_bits is not None:
        u = to_device_bf16(up_bits, device)
        t = nv.nvfp4_quantize_swiglu(x, u, m=m)
    else:
        t = nv.nvfp4_quantize(x, rows=m)
    import torch
    torch.cuda.synchronize(device)
    return t, t.qdata.cpu().numpy(), t.scales.cpu().numpy(), float(t.global_scale.item())
