"""Seeded input generators (no GPU)."""
import numpy as np

from roofline_driven_optimisation_amd.inputs import (bf16_bits_to_f32, f32_to_bf16_bits,
                                                     make_case, workload)


def test_deterministic_and_ordered():
    a = make_case(5, 6, 7, "f32", 1.5, 0.5, seed=0)
    b = make_case(5, 6, 7, "f32", 1.5, 0.5, seed=0)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.B, b.B) and np.array_equal(a.C, b.C)
    # A is drawn first, then B, then C, from one generator
    rng = np.random.default_rng(0)
    A = rng.uniform(-1, 1, (5, 7)).astype(np.float32)
    B = rng.uniform(-1, 1, (7, 6)).astype(np.float32)
    C = rng.uniform(-1, 1, (5, 6)).astype(np.float32)
    assert np.array_equal(a.A, A) and np.array_equal(a.B, B) and np.array_equal(a.C, C)


def test_beta_zero_has_no_c():
    assert make_case(3, 3, 3, "f32", 1.0, 0.0).C is None


def test_bf16_case_bits():
    c = make_case(4, 8, 16, "bf16", dist_a="n:1.0", dist_b="n:0.02")
    assert c.A.dtype == np.uint16 and c.B.dtype == np.uint16
    wide = bf16_bits_to_f32(c.A)
    # widening then rounding again is the identity
    assert np.array_equal(f32_to_bf16_bits(wide), c.A)


def test_rne_ties():
    # 1 + 2^-8 lies exactly between bf16 1.0 and 1.0078125: ties to even (1.0)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert got[0] == 1.0 and got[1] == 1.0 + 4 * 2 ** -8


def test_integer_distribution_exact():
    c = make_case(16, 16, 16, "bf16", dist_a="i:4", dist_b="i:4")
    v = bf16_bits_to_f32(c.A)
    assert np.all(v == np.round(v)) and np.abs(v).max() <= 4


def test_workload_distributions():
    w = workload("bf16_4096")
    c = make_case(64, 64, 4096, w.dtype, dist_a=w.dist_a, dist_b=w.dist_b)
    std = bf16_bits_to_f32(c.A).std()
    assert abs(std - 1 / 64) < 1e-3
