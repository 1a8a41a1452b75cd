"""The seeded input generator: splitmix64 conformance, determinism, prefix stability,
outlier channels and distribution shape of the synthetic workloads."""
import numpy as np

import synth

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def py_mix64(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def test_splitmix64_published_first_output():
    # splitmix64 seeded with 0 returns 0xe220a8397b1dcdaf first (Vigna's reference generator)
    assert py_mix64(GOLDEN) == 0xE220A8397B1DCDAF


def test_draw_is_splitmix64_stream():
    for seed, tag in [(0, 1), (440420, 2), (7, 31)]:
        key = py_mix64((seed * GOLDEN + py_mix64(tag + 1)) & MASK64)
        for i in [0, 1, 2, 1000, 123456789]:
            assert synth.draw(seed, tag, i) == py_mix64((key + (i + 1) * GOLDEN) & MASK64)


def test_deterministic_and_prefix_stable():
    a = synth.normal_bf16(64, 96, seed=1, tag=2, sigma=1.0)
    b = synth.normal_bf16(64, 96, seed=1, tag=2, sigma=1.0, threads=1)
    c = synth.normal_bf16(17, 96, seed=1, tag=2, sigma=1.0)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a[:17], c)
    d = synth.normal_bf16(64, 96, seed=1, tag=3, sigma=1.0)
    assert (a != d).mean() > 0.9


def test_outlier_channels():
    w = synth.FC2
    assert w.n_outliers == 143
    mask = w.mask()
    assert mask.sum() == 143
    np.testing.assert_array_equal(mask, w.mask())
    x = synth.normal_bf16(512, w.k, seed=w.seed, tag=synth.TAG_GATE, sigma=1.0, mask=mask)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    std_out = f[:, mask == 1].std()
    std_in = f[:, mask == 0].std()
    assert 18 < std_out / std_in < 22
    assert 0.97 < std_in < 1.03


def test_weight_distribution():
    w = synth.TINY
    f = (w.weight().astype(np.uint32) << 16).view(np.float32)
    assert abs(f.std() - 0.02) < 0.001
    assert abs(f.mean()) < 0.001


def test_workload_table():
    assert synth.FC2.m_pad == 37824
    assert [w.m_pad for w in synth.RAGGED] == [37712, 37728, 37744, 37776, 37824, 37840, 37968, 38224]
    assert [w.seed for w in synth.RAGGED] == list(range(100, 108))
    assert synth.TINY.m_pad == 256
    assert abs(synth.FC2.gemm_flops - 5.828e12) / 5.828e12 < 1e-3
