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


def pin_epilogue_closed_forms(o):
    """Activations against closed forms and independent library routines:
    ReLU by sign; GELU(x) = x * Phi(x) with Phi from scipy.special.ndtr and
    the table value Phi(1) = 0.8413447460685429; SiLU(x) = x * expit(x);
    for both, f(x) - f(-x) = x (since Phi(x) + Phi(-x) = 1 and likewise for
    the logistic function)."""
    from scipy.special import expit, ndtr
    x = np.array([[-6.0, -3.0, -1.0, -0.5, 0.0, 0.25, 1.0, 2.5, 7.0]])
    one = np.ones_like(x)
    y, _ = o.epilogue(x, one, None, 1)
    assert np.array_equal(y, np.where(x < 0, 0.0, x))
    y, _ = o.epilogue(x, one, None, 2)
    assert np.allclose(y, x * ndtr(x), rtol=1e-14, atol=1e-300)
    assert abs(o.epilogue(np.array([[1.0]]), np.ones((1, 1)), None, 2)[0][0, 0]
               - 0.8413447460685429) < 1e-15
    yn, _ = o.epilogue(-x, one, None, 2)
    assert np.allclose(y - yn, x, rtol=1e-14, atol=1e-14)
    y, _ = o.epilogue(x, one, None, 3)
    assert np.allclose(y, x * expit(x), rtol=1e-14, atol=1e-300)
    yn, _ = o.epilogue(-x, one, None, 3)
    assert np.allclose(y - yn, x, rtol=1e-14, atol=1e-14)
    y, _ = o.epilogue(x, one, None, 0)
    assert np.array_equal(y, x)


def pin_epilogue_bias_columns(o):
    """The bias vector runs along the N columns of a row-major result, and
    the denominator grows by |bias[n]|."""
    z = np.arange(15, dtype=np.float64).reshape(3, 5) - 7.0
    den = np.full_like(z, 2.0)
    bias = np.array([0.5, -1.0, 2.0, -4.0, 8.0], dtype=np.float32)
    y, d = o.epilogue(z, den, bias, 0)
    assert np.array_equal(y, z + bias.astype(np.float64)[None, :])
    assert np.array_equal(d, den + np.abs(bias.astype(np.float64))[None, :])
    y, d = o.epilogue(z[1], den[1], bias, 1, cols=np.arange(5))
    assert np.array_equal(y, np.maximum(z[1] + bias, 0.0))


def pin_epilogue_gemm(o):
    """Through gemm(): K = 0 gives act(beta * C + bias); the fused result of
    a small integer product equals the epilogue applied to the plain one; and
    sampled entries agree with the full matrix."""
    C = _mat([[1, -2, 3], [-4, 5, -6]])
    bias = np.array([1.0, 1.5, -2.0], dtype=np.float32)
    y, _ = o.gemm(np.zeros((2, 0), np.float32), np.zeros((0, 3), np.float32), C, 1.0, 0.5,
                  bias=bias, act=1)
    assert np.array_equal(y, np.maximum(0.5 * C.astype(np.float64) + bias, 0.0))
    A = _mat([[1, 2], [3, -4]])
    B = _mat([[5, -6, 7], [8, 9, -1]])
    z, den = o.gemm(A, B)
    y, d = o.gemm(A, B, bias=bias, act=3)
    y2, d2 = o.epilogue(z, den, bias, 3)
    assert np.array_equal(y, y2) and np.array_equal(d, d2)
    rows, cols = np.array([1, 0, 1]), np.array([2, 0, 1])
    ye, de = o.gemm_entries(A, B, rows, cols, bias=bias, act=2)
    yf, df = o.gemm(A, B, bias=bias, act=2)
    assert np.array_equal(ye, yf[rows, cols]) and np.array_equal(de, df[rows, cols])


def pin_epilogue_slope(o):
    """The denominator's slope factor bounds |act'| everywhere: GELU' =
    Phi(x) + x phi(x) and SiLU' = s(x) (1 + x (1 - s(x))) on a fine grid stay
    below the factors 1.13 and 1.10 the oracle applies (1 for ReLU)."""
    from scipy.special import expit, ndtr
    x = np.linspace(-20, 20, 400001)
    gelu_d = ndtr(x) + x * np.exp(-x * x / 2) / np.sqrt(2 * np.pi)
    s = expit(x)
    silu_d = s * (1 + x * (1 - s))
    one = np.ones((1, 1))
    for act, deriv in [(2, gelu_d), (3, silu_d)]:
        _, d = o.epilogue(np.zeros((1, 1)), one, None, act)
        assert np.max(np.abs(deriv)) <= d[0, 0] < np.max(np.abs(deriv)) + 0.01, act
    _, d = o.epilogue(np.zeros((1, 1)), one, None, 1)
    assert d[0, 0] == 1.0


def pin_sum_closed_forms(o):
    """Vector sum: Gauss's n (n - 1) / 2 for 0 .. n-1, n for ones, the empty
    sum, alternating signs, and magnitudes summing to sum |x|."""
    for n in (1, 2, 7, 1000, 4097):
        x = np.arange(n, dtype=np.float32)
        s, a = o.sum_f32(x)
        assert s == n * (n - 1) / 2 and a == s
        s, a = o.sum_f32(np.ones(n, np.float32))
        assert s == n and a == n
        alt = np.where(np.arange(n) % 2 == 0, 1.0, -1.0).astype(np.float32)
        s, a = o.sum_f32(alt)
        assert s == (n % 2) and a == n
    assert o.sum_f32(np.zeros(0, np.float32)) == (0.0, 0.0)


def pin_sum_precision(o):
    """fp64 accumulation: 1e8 + 1 - 1e8 is 1 (an fp32 accumulator loses the
    1); random data agrees with math.fsum (exactly rounded) to fp64
    rounding."""
    import math
    s, a = o.sum_f32(np.array([1e8, 1.0, -1e8], dtype=np.float32))
    assert s == 1.0 and a == 2e8 + 1
    rng = np.random.default_rng(11)
    x = rng.uniform(-1, 1, 100003).astype(np.float32)
    s, a = o.sum_f32(x)
    ref = math.fsum(x.astype(np.float64))
    assert abs(s - ref) <= 1e-12 * math.fsum(np.abs(x.astype(np.float64)))
    assert abs(a - math.fsum(np.abs(x.astype(np.float64)))) <= 1e-12 * a


def pin_batched(o):
    """Strided batched form: a stored transpose with trans_b equals the plain
    product (the indexing of B^T), every item equals its own single GEMM
    on hand values, and items do not mix."""
    A = np.stack([_mat([[1, 2], [3, 4]]), _mat([[0, 1], [1, 0]])])
    B = np.stack([_mat([[5, 6, 7], [8, 9, 10]]), _mat([[1, 2, 3], [4, 5, 6]])])
    got, _ = o.gemm_batched(A, B)
    assert np.array_equal(got[0], [[21, 24, 27], [47, 54, 61]])
    assert np.array_equal(got[1], [[4, 5, 6], [1, 2, 3]])  # a row swap
    Bt = np.ascontiguousarray(np.transpose(B, (0, 2, 1)))
    got_t, _ = o.gemm_batched(A, Bt, trans_b=True)
    assert np.array_equal(got_t, got)
    C = np.stack([_mat([[1, 1, 1], [1, 1, 1]]), _mat([[2, 0, 2], [0, 2, 0]])])
    got_c, _ = o.gemm_batched(A, Bt, C, alpha=2.0, beta=0.5, trans_b=True)
    assert np.array_equal(got_c, 2.0 * got + 0.5 * C.astype(np.float64))


def pin_fp8(o):
    """8-bit floats: table values of both formats (E4M3 1, 2, -1, the largest
    448, the smallest subnormal 2^-9, NaN; E5M2 the largest 57344, 2^-16,
    infinity); every finite code survives encode-decode; the fp8 GEMM equals
    the plain GEMM on the decoded values with B transposed, scales folded
    into alpha."""
    from roofline_driven_optimisation_amd.inputs import f32_to_fp8_bits
    d = o.fp8_decode(np.array([0x38, 0x40, 0xB8, 0x7E, 0x01, 0x7F], np.uint8), 0)
    assert list(d[:5]) == [1.0, 2.0, -1.0, 448.0, 2.0 ** -9] and np.isnan(d[5])
    d = o.fp8_decode(np.array([0x3C, 0x7B, 0x01, 0x7C, 0xFC], np.uint8), 1)
    assert list(d) == [1.0, 57344.0, 2.0 ** -16, np.inf, -np.inf]
    for fmt, nan in ((0, lambda b: (b & 0x7F) == 0x7F), (1, lambda b: (b & 0x7C) == 0x7C)):
        codes = np.array([b for b in range(256) if not nan(b) and b != 0x80], np.uint8)
        vals = o.fp8_decode(codes, fmt)
        assert np.array_equal(f32_to_fp8_bits(vals.astype(np.float32), fmt), codes)
        # halfway between 1 and the next code rounds to the even code (1)
        step = 2.0 ** (-3 if fmt == 0 else -2)
        assert f32_to_fp8_bits(np.array([1 + step / 2], np.float32), fmt)[0] == (0x38 if fmt == 0 else 0x3C)
    rng = np.random.default_rng(12)
    A = f32_to_fp8_bits(rng.standard_normal((9, 40)).astype(np.float32), 0)
    Bt = f32_to_fp8_bits(rng.standard_normal((7, 40)).astype(np.float32), 0)
    C = rng.standard_normal((9, 7)).astype(np.float32)
    got, den = o.gemm_fp8(A, Bt, C, alpha=1.5, beta=0.5, sa=0.25, sb=2.0, fmt=0)
    Af = o.fp8_decode(A, 0).astype(np.float32)
    Bf = np.ascontiguousarray(o.fp8_decode(Bt, 0).T).astype(np.float32)
    ref, rden = o.gemm(Af, Bf, C, alpha=1.5 * 0.25 * 2.0, beta=0.5)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-14) and np.allclose(den, rden, rtol=1e-14)


ALL_PINS = [
    pin_hand_signs, pin_rectangular_hand, pin_identity_zero_permutation, pin_all_ones,
    pin_alpha_beta_linearity, pin_transpose_identity, pin_brute_force_integers,
    pin_random_floats_vs_numpy, pin_bf16_widening, pin_beta_zero_reads_no_c, pin_k_zero,
    pin_entries_match_full, pin_entries_hand, pin_den_bounds_result,
    pin_epilogue_closed_forms, pin_epilogue_bias_columns, pin_epilogue_gemm, pin_epilogue_slope,
    pin_sum_closed_forms, pin_sum_precision, pin_batched, pin_fp8,
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
    "bias_by_row": ("int64_t n = cols != NULL ? cols[e] : e % N;",
                    "int64_t n = cols != NULL ? cols[e] : (e / N) % N;"),
    "bias_dropped": ("y[e] = act_fn(act, z[e] + b);", "y[e] = act_fn(act, z[e]);"),
    "den_without_bias": ("den_out[e] = slope * (den[e] + fabs(b));", "den_out[e] = slope * den[e];"),
    "slope_dropped": ("return act == 2 ? 1.13 : act == 3 ? 1.10 : 1.0;", "return 1.0;"),
    "gelu_unscaled_erf": ("erfc(-x / sqrt(2.0))", "erfc(-x)"),
    "silu_sign": ("x / (1.0 + exp(-x))", "x / (1.0 + exp(x))"),
    "relu_leaky": ("return x < 0.0 ? 0.0 : x;", "return x < 0.0 ? 0.01 * x : x;"),
    "sum_skips_first": ("for (int64_t i = 0; i < n; ++i) {\n        s += (double)x[i];",
                        "for (int64_t i = 1; i < n; ++i) {\n        s += (double)x[i];"),
    "sum_in_float": ("double s = 0.0, a = 0.0;", "float s = 0.0f; double a = 0.0;"),
    "abs_sum_signed": ("a += fabs((double)x[i]);", "a += (double)x[i];"),
    "fp8_e4m3_bias": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "fp8_e5m2_mantissa": ("ldexp(1.0 + m / 4.0, e - 15)", "ldexp(1.0 + m / 8.0, e - 15)"),
    "fp8_b_not_transposed": ("fp8_value(B[n * K + k], fmt)", "fp8_value(B[k * N + n], fmt)"),
    "fp8_scale_dropped": ("const double scale = alpha * sa * sb;", "const double scale = alpha * sa;"),
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
