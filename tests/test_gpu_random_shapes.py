"""GPU parity of the whole path on seeded random shapes: the SwiGLU producer, the
plain weight quantizer and the GEMM against the CPU oracle on every element, with
tails in all three dimensions (M any positive size, N a multiple of 16, K a multiple
of 64, so half K steps occur). The shapes are drawn once from a fixed seed, so every
run checks the same ones."""
import random

import pytest

import synth
from tests.test_gpu_gemm import run_path

pytestmark = pytest.mark.gpu


def _shapes(count=10, seed=2026):
    r = random.Random(seed)
    out = []
    for _ in range(count):
        m = r.randint(1, 1200)
        n = 16 * r.randint(1, 64)
        k = 64 * r.randint(1, 32)
        out.append((m, n, k))
    return out


@pytest.mark.parametrize("m,n,k", _shapes())
def test_random_shape_full_path(gpu, m, n, k):
    w = synth.Workload(f"random_{m}x{n}x{k}", m=m, n=n, k=k, seed=m * 7 + n * 3 + k, swiglu=True,
                       outliers=(m + n) % 2 == 0)
    _, st = run_path(w, gpu, None, 0)
    assert st["checked"] == synth.padded_rows(m) * n
