"""Pin functions for the CPU oracle, shared by the tests and by the
planted-mistake children (each runs in a fresh interpreter).

Each pin ties the oracle to something other than itself: values the pages
print, closed forms, exact identities, and an independent fp64 path (numpy's
float64 matmul) on inputs where every product and sum is exact.
"""
import numpy as np

from roofline_driven_optimisation_amd.inputs import f32_to_bf16_bits, make_case


def _mat(rows):
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float32)


# ---------------------------------------------------------------------------
# pin functions: each takes an Oracle and raises AssertionError on a mismatch
# ---------------------------------------------------------------------------

def pin_worked_2x2(o, golden_sections):
    """Page "From model computation to GPU execution", section 4.3."""
    A, B, C = (_mat(golden_sections[k]) for k in ("A", "B", "C"))
    Cref, den = o.gemm(A, B)
    assert np.array_equal(Cref, C.astype(np.float64))
    Cref16, _ = o.gemm(f32_to_bf16_bits(A), f32_to_bf16_bits(B), bf16=True)
    assert np.array_equal(Cref16, C.astype(np.float64))
    # with |products| all positive the denominator equals the result
    assert np.allclose(den, C, rtol=0, atol=1e-12)


def pin_hand_signs(o):
    """A hand-computed case with mixed signs, alpha and beta.

    A = [[1, -2, 3]], B = [[4], [5], [-6]], C_in = [[8]], alpha = 2, beta = -0.5:
    sum = 4 - 10 - 18 = -24; C = 2*(-24) - 0.5*8 = -52;
    den = 2*(4 + 10 + 18) + |-0.5*8| = 68.
    """
    A = _mat([[1, -2, 3]])
    B = _mat([[4], [5], [-6]])
    C = _mat([[8]])
    Cref, den = o.gemm(A, B, C, alpha=2.0, beta=-0.5)
    assert Cref[0, 0] == -52.0
    assert abs(den[0, 0] - 68.0) < 1e-12


def pin_rectangular_hand(o):
    """A 2x3 times 3x2 product written out by hand (catches transposed
    indexing of either operand on a non-square shape)."""
    A = _mat([[1, 2, 3], [4, 5, 6]])
    B = _mat([[7, 8], [9, 10], [11, 12]])
    # row 0: 7+18+33=58, 8+20+36=64; row 1: 28+45+66=139, 32+50+72=154
    Cref, _ = o.gemm(A, B)
    assert np.array_equal(Cref, np.array([[58, 64], [139, 154]], dtype=np.float64))


def pin_identity_zero_permutation(o):
    rng = np.random.default_rng(1)
    A = rng.uniform(-1, 1, (7, 5)).astype(np.float32)
    B = rng.uniform(-1, 1, (5, 9)).astype(np.float32)
    I5 = np.eye(5, dtype=np.float32)
    I7 = np.eye(7, dtype=np.float32)
    assert np.array_equal(o.gemm(A, I5)[0], A.astype(np.float64))
    assert np.array_equal(o.gemm(I7, A)[0], A.astype(np.float64))
    assert np.array_equal(o.gemm(np.zeros((7, 5), np.float32), B)[0], np.zeros((7, 9)))
    perm = np.array([3, 0, 4, 1, 2])
    P = np.eye(5, dtype=np.float32)[perm]  # (P B)[i] = B[perm[i]]
    assert np.array_equal(o.gemm(P, B)[0], B[perm].astype(np.float64))
    Q = np.eye(5, dtype=np.float32)[:, perm]  # (A Q)[:, j] = A[:, perm[j]]
    assert np.array_equal(o.gemm(A, Q)[0], A[:, perm].astype(np.float64))


def pin_all_ones(o):
    """A = B = ones gives sum K; C = alpha*K + beta*C_in exactly."""
    for (M, N, K) in [(1, 1, 1), (3, 4, 5), (17, 9, 33)]:
        C = np.arange(M * N, dtype=np.float32).reshape(M, N) - 3
        Cref, den = o.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32), C,
                           alpha=1.5, beta=0.5)
        assert np.array_equal(Cref, 1.5 * K + 0.5 * C.astype(np.float64))
        assert np.allclose(den, 1.5 * K + np.abs(0.5 * C), rtol=0, atol=1e-12)


def pin_alpha_beta_linearity(o):
    rng = np.random.default_rng(2)
    A = rng.integers(-4, 5, (6, 11)).astype(np.float32)
    B = rng.integers(-4, 5, (11, 5)).astype(np.float32)
    C = rng.integers(-4, 5, (6, 5)).astype(np.float32)
    base, _ = o.gemm(A, B)
    for alpha, beta in [(1.5, 0.5), (-2.0, 3.0), (0.0, 1.0), (1.0, -1.0)]:
        got, _ = o.gemm(A, B, C, alpha=alpha, beta=beta)
        assert np.array_equal(got, alpha * base + beta * C.astype(np.float64))


def pin_transpose_identity(o):
    """(A B)^T = B^T A^T, exact on integer data."""
    rng = np.random.default_rng(3)
    for (M, N, K) in [(5, 7, 3), (13, 2, 17), (1, 9, 4)]:
        A = rng.integers(-4, 5, (M, K)).astype(np.float32)
        B = rng.integers(-4, 5, (K, N)).astype(np.float32)
        AB, _ = o.gemm(A, B)
        BtAt, _ = o.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
        assert np.array_equal(AB.T, BtAt)


def pin_brute_force_integers(o):
    """Integer entries in [-4, 4]: every partial sum is exact in fp64, so the
    oracle must equal numpy's float64 matmul bit for bit, on odd sizes."""
    rng = np.random.default_rng(4)
    for (M, N, K) in [(1, 1, 1), (1, 64, 3), (64, 1, 5), (3, 5, 7), (17, 33, 65), (31, 29, 64)]:
        for bf16 in (False, True):
            A = rng.integers(-4, 5, (M, K)).astype(np.float32)
            B = rng.integers(-4, 5, (K, N)).astype(np.float32)
            C = rng.integers(-4, 5, (M, N)).astype(np.float32)
            ref = 1.5 * (A.astype(np.float64) @ B.astype(np.float64)) + 0.5 * C
            if bf16:
                got, _ = o.gemm(f32_to_bf16_bits(A), f32_to_bf16_bits(B), C, 1.5, 0.5, bf16=True)
            else:
                got, _ = o.gemm(A, B, C, 1.5, 0.5)
            assert np.array_equal(got, ref), (M, N, K, bf16)


def pin_random_floats_vs_numpy(o):
    """Random floats: agreement with numpy float64 matmul to fp64 rounding."""
    rng = np.random.default_rng(5)
    for (M, N, K) in [(8, 8, 8), (37, 41, 129), (64, 3, 500)]:
        A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        got, den = o.gemm(A, B)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        assert np.max(np.abs(got - ref) / den) < 1e-13


def pin_bf16_widening(o):
    """Known bf16 bit patterns are widened exactly: 0x3F80=1, 0xC000=-2,
    0x4049=3.140625, 0x3F00=0.5, 0x0001 = 2^-133 (smallest subnormal)."""
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x3F00: 0.5, 0x0001: 2.0 ** -133}
    one = np.array([[0x3F80]], dtype=np.uint16)
    for bits, val in cases.items():
        got, _ = o.gemm(np.array([[bits]], dtype=np.uint16), one, bf16=True)
        assert got[0, 0] == val, hex(bits)


def pin_beta_zero_reads_no_c(o):
    A = _mat([[1, 2]])
    B = _mat([[3], [4]])
    C = np.full((1, 1), np.nan, dtype=np.float32)
    got, den = o.gemm(A, B, C, alpha=1.0, beta=0.0)
    assert got[0, 0] == 11.0 and np.isfinite(den[0, 0])


def pin_k_zero(o):
    C = _mat([[1, -2], [3, 4]])
    got, _ = o.gemm(np.zeros((2, 0), np.float32), np.zeros((0, 2), np.float32), C,
                    alpha=1.5, beta=0.5)
    assert np.array_equal(got, 0.5 * C.astype(np.float64))
    got0, _ = o.gemm(np.zeros((2, 0), np.float32), np.zeros((0, 2), np.float32))
    assert np.array_equal(got0, np.zeros((2, 2)))


def pin_entries_match_full(o):
    case = make_case(23, 19, 37, "bf16", 1.5, 0.5, "n:0.3", "n:0.3", "u", seed=6)
    full, fden = o.gemm(case.A, case.B, case.C, 1.5, 0.5, bf16=True)
    rows = np.array([0, 22, 5, 11, 22])
    cols = np.array([0, 18, 7, 0, 3])
    got, den = o.gemm_entries(case.A, case.B, rows, cols, case.C, 1.5, 0.5, bf16=True)
    assert np.array_equal(got, full[rows, cols])
    assert np.array_equal(den, fden[rows, cols])


def pin_entries_hand(o):
    """The sampled-entry path on its own: the worked 2x2 product."""
    A = _mat([[1, 2], [3, 4]])
    B = _mat([[5, 6], [7, 8]])
    got, _ = o.gemm_entries(A, B, [1, 0, 1], [0, 1, 1])
    assert list(got) == [43.0, 22.0, 50.0]
    got, _ = o.gemm_entries(A, B, [1], [0], C=_mat([[0, 0], [10, 0]]), alpha=2.0, beta=0.5)
    assert list(got) == [91.0]


def pin_den_bounds_result(o):
    """Triangle inequality: |C_ref| <= den, with equality for nonnegative data."""
    rng = np.random.default_rng(7)
    A = rng.normal(size=(9, 13)).astype(np.float32)
    B = rng.normal(size=(13, 6)).astype(np.float32)
    C = rng.normal(size=(9, 6)).astype(np.float32)
    got, den = o.gemm(A, B, C, -1.5, 0.25)
    assert np.all(np.abs(got) <= den * (1 + 1e-15))
    got, den = o.gemm(np.abs(A), np.abs(B))
    assert np.allclose(got, den, rtol=1e-15, atol=1e-29)


ALL_PINS = [
    pin_hand_signs, pin_rectangular_hand, pin_identity_zero_permutation, pin_all_ones,
    pin_alpha_beta_linearity, pin_transpose_identity, pin_brute_force_integers,
    pin_random_floats_vs_numpy, pin_bf16_widening, pin_beta_zero_reads_no_c, pin_k_zero,
    pin_entries_match_full, pin_entries_hand, pin_den_bounds_result,
]


# Plausible mistakes planted into copies of the oracle's C source; every one
# must make at least one pin fail.
MUTANTS = {
    "b_index_transposed": ("load_elem(B, kind, k * N + n)", "load_elem(B, kind, n * K + k)"),
    "a_index_transposed": ("load_elem(A, kind, m * K + k);", "load_elem(A, kind, k * M + m);"),
    "dropped_beta": ("acc[n] = alpha * acc[n] + beta * c_in;", "acc[n] = alpha * acc[n];"),
    "alpha_on_c": ("acc[n] = alpha * acc[n] + beta * c_in;",
                   "acc[n] = alpha * (acc[n] + beta * c_in);"),
    "sign_flip": ("acc[n] += p;", "acc[n] -= p;"),
    "den_without_abs": ("mag[n] += fabs(p);", "mag[n] += p;"),
    "den_without_beta": ("+ fabs(beta * c_in) + 1e-30;\n        }", "+ 1e-30;\n        }"),
    "k_off_by_one": ("for (int64_t k = 0; k < K; ++k) {\n            double a",
                     "for (int64_t k = 1; k < K; ++k) {\n            double a"),
    "bf16_wrong_shift": ("<< 16;", "<< 15;"),
    "beta_reads_c_always": ("double c_in = (beta != 0.0) ? (double)Cin[m * N + n] : 0.0;\n            acc",
                            "double c_in = (double)Cin[m * N + n];\n            acc"),
    "entries_b_transposed": ("load_elem(B, kind, k * N + n);\n            acc +=",
                             "load_elem(B, kind, n * K + k);\n            acc +="),
    "entries_dropped_alpha": ("out[e] = alpha * acc + beta * c_in;", "out[e] = acc + beta * c_in;"),
}


def _run_pins(o, golden_sections):
    failures = []
    for pin in [lambda x: pin_worked_2x2(x, golden_sections)] + ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, OSError):
            failures.append(getattr(pin, "__name__", "worked_2x2"))
        except Exception as exc:  # a crash in the mutant counts as caught
            failures.append(repr(exc))
    return failures




def main(lib_path, golden_path):
    """Child entry: run every pin on one compiled library, print the failures."""
    import json
    import sys

    sys.path.insert(0, __import__("os").path.dirname(__file__))
    from conftest import read_golden_path
    from oracle import Oracle
    failures = _run_pins(Oracle(lib_path), read_golden_path(golden_path))
    print("PIN_FAILURES " + json.dumps(failures))
