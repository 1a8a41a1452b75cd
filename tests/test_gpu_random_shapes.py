"""GPU parity on seeded random shapes, against the CPU oracle on every element, with
tails in every dimension (M any positive size, N a multiple of 16, K a multiple of 64,
so half K steps occur): the whole path (SwiGLU producer, weight quantizer, GEMM), the
GEMM with bias and gated residual, the SwiGLU-pair GEMM, the modulated producer and
the single-read producers. The shapes are drawn once from fixed seeds, so every run
checks the same ones."""
import random

import pytest

import synth
from tests import test_gpu_gemm_fused as fused
from tests import test_gpu_gemm_swiglu as pair
from tests import test_gpu_producer_amax as single_read
from tests import test_gpu_producer_modulate as modulate
from tests.test_gpu_gemm import run_path

pytestmark = pytest.mark.gpu


def _shapes(count=10, seed=2026, m_max=1200, n16_max=64, k64_max=32):
    r = random.Random(seed)
    out = []
    for _ in range(count):
        m = r.randint(1, m_max)
        n = 16 * r.randint(1, n16_max)
        k = 64 * r.randint(1, k64_max)
        out.append((m, n, k))
    return out


@pytest.mark.parametrize("m,n,k", _shapes())
def test_random_shape_full_path(gpu, m, n, k):
    w = synth.Workload(f"random_{m}x{n}x{k}", m=m, n=n, k=k, seed=m * 7 + n * 3 + k, swiglu=True,
                       outliers=(m + n) % 2 == 0)
    _, st = run_path(w, gpu, None, 0)
    assert st["checked"] == synth.padded_rows(m) * n


@pytest.mark.parametrize("m,n,k", _shapes(6, seed=2027, m_max=700, n16_max=40, k64_max=20))
def test_random_shape_bias_and_gated_residual(gpu, m, n, k):
    fused.check_bias_and_gated_residual(gpu, m, n, k)


@pytest.mark.parametrize("m,n,k", _shapes(6, seed=2028, m_max=700, n16_max=40, k64_max=20))
def test_random_shape_swiglu_pair(gpu, m, n, k):
    pair.check_pair(gpu, m, n // 2, k)


@pytest.mark.parametrize("m,_n,k", _shapes(8, seed=2029, m_max=2000, k64_max=48))
def test_random_shape_modulated_producer(gpu, m, _n, k):
    x = synth.normal_bf16(m, k, seed=m + k, tag=1, sigma=1.0)
    sc, sh = modulate.vectors(k, m + 3)
    modulate.check_mod(x, sc, sh, gpu, f"random m={m} k={k}")


@pytest.mark.parametrize("m,_n,k", _shapes(8, seed=2030, m_max=2000, k64_max=48))
def test_random_shape_single_read_producers(gpu, m, _n, k):
    gate = synth.normal_bf16(m, k, seed=m + 2 * k, tag=1, sigma=1.0)
    up = synth.normal_bf16(m, k, seed=m + 2 * k, tag=2, sigma=1.0)
    single_read.check_amax(gate, up, single_read.true_amax(gate, up), gpu, f"random swiglu m={m} k={k}")
    single_read.check_amax(gate, None, single_read.true_amax(gate, None), gpu, f"random plain m={m} k={k}")
