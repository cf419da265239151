"""The seeded input generator: deterministic, and its bf16 encoding rounds to
nearest-even."""
import numpy as np

from matrix_optimizer_amd import workloads as WL


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20, 0.0], np.float32)
    bits = WL.f32_to_bf16_bits(x)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 ties -> 1+2^-6 (even mantissa)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81, 0x0000]
    assert np.array_equal(WL.bf16_bits_to_f32(bits), np.array([1, 1, 1 + 2 ** -6, -2.5, 1 + 2 ** -7, 0], np.float32))


def test_deterministic_and_independent_matrices():
    w = WL.WORKLOADS["moe_experts"]
    a = w.matrix(0, 3, "grad")
    b = w.matrix(0, 3, "grad")
    assert a.dtype == np.uint16 and a.shape == (24, 10240)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, w.matrix(0, 4, "grad"))
    assert np.all(w.matrix(0, 3, "momentum") == 0)


def test_single_matrix_recipe():
    w = WL.WORKLOADS["single_128x256_f32"]
    rng = np.random.default_rng(0)
    g = rng.standard_normal((128, 256))
    m = rng.standard_normal((128, 256))
    p = rng.normal(0.0, 0.02, (128, 256))
    assert np.array_equal(w.matrix(0, 0, "grad"), g.astype(np.float32))
    assert np.array_equal(w.matrix(0, 0, "momentum"), m.astype(np.float32))
    assert np.array_equal(w.matrix(0, 0, "param"), p.astype(np.float32))


def test_nominal_flops():
    w = WL.WORKLOADS["fused_74x24x10240"]
    assert w.nominal_ns_flops() == 74 * 5 * (4 * 24 * 24 * 10240 + 2 * 24 ** 3)
