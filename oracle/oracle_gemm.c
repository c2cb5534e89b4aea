/*
 * CPU oracle for the general matrix multiply  C = alpha * A * B + beta * C.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * GPU library.
 *
 * What it computes (page "Naive GEMM and Roofline analysis", section 10.1,
 * the GEMM definition): for every output row m and column n,
 *
 *     C_ref[m][n] = alpha * sum_{k=0}^{K-1} A[m][k] * B[k][n] + beta * C_in[m][n]
 *
 * with A, B and C stored densely row-major, A[m][k] at m*K+k, B[k][n] at
 * k*N+n and C[m][n] at m*N+n, exactly the indexing of the naive kernel in
 * section 10.2 of the same page.  The worked 2x2 example of page "From model
 * computation to GPU execution", section 4.3, is the same dot-product view.
 *
 * Arithmetic is fp64 throughout: inputs are widened exactly (fp32 -> double,
 * or a bf16 bit pattern -> fp32 -> double), the sum over k runs in ascending
 * k order, and the result is kept in fp64, never rounded.  Beside each result
 * the oracle returns the error denominator used by the parity tests,
 *
 *     den[m][n] = |alpha| * sum_k |A[m][k] * B[k][n]| + |beta * C_in[m][n]| + 1e-30,
 *
 * so that a GPU value c passes when |c - C_ref| / den is within tolerance.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - beta == 0: C_in is not read at all (it may be NULL or hold NaN); the
 *     GEMM section of page "Where kernel performance comes from" assumes the
 *     old C need not be read when beta is zero.
 *   - K == 0: the sum is empty, so C_ref = beta * C_in (zeros when beta == 0).
 *   - M == 0 or N == 0: nothing to do.
 *
 * The only parallelism is an OpenMP loop over independent output rows (or
 * independent sampled entries); each row is the plain i-k-j triple loop.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

enum { ELEM_F32 = 0, ELEM_BF16 = 1 };

/* Exact widening of one stored element to double. */
static double load_elem(const void *base, int kind, int64_t idx)
{
    if (kind == ELEM_F32)
        return (double)((const float *)base)[idx];
    /* bf16 is the upper 16 bits of an IEEE binary32 value. */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int check_args(int64_t M, int64_t N, int64_t K, double beta,
                      const void *A, const void *B, const float *Cin,
                      const double *Cref, const double *den)
{
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_EINVAL;
    if (M > 0 && K > 0 && A == NULL)
        return ORACLE_EINVAL;
    if (K > 0 && N > 0 && B == NULL)
        return ORACLE_EINVAL;
    if (M > 0 && N > 0 && (Cref == NULL || den == NULL))
        return ORACLE_EINVAL;
    if (M > 0 && N > 0 && beta != 0.0 && Cin == NULL)
        return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* Full output: every (m, n), row by row, i-k-j order. */
static int gemm_full(int64_t M, int64_t N, int64_t K, double alpha, double beta,
                     const void *A, const void *B, int kind, const float *Cin,
                     double *Cref, double *den)
{
    int rc = check_args(M, N, K, beta, A, B, Cin, Cref, den);
    if (rc != ORACLE_OK || M == 0 || N == 0)
        return rc;

    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        double *acc = Cref + m * N; /* running sum over k   */
        double *mag = den + m * N;  /* running sum of |A*B| */
        for (int64_t n = 0; n < N; ++n) {
            acc[n] = 0.0;
            mag[n] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            double a = load_elem(A, kind, m * K + k);
            for (int64_t n = 0; n < N; ++n) {
                double p = a * load_elem(B, kind, k * N + n);
                acc[n] += p;
                mag[n] += fabs(p);
            }
        }
        for (int64_t n = 0; n < N; ++n) {
            double c_in = (beta != 0.0) ? (double)Cin[m * N + n] : 0.0;
            acc[n] = alpha * acc[n] + beta * c_in;
            mag[n] = fabs(alpha) * mag[n] + fabs(beta * c_in) + 1e-30;
        }
    }
    return ORACLE_OK;
}

/* Selected outputs only: entry e is (rows[e], cols[e]); one dot product each. */
static int gemm_entries(int64_t M, int64_t N, int64_t K, double alpha, double beta,
                        const void *A, const void *B, int kind, const float *Cin,
                        int64_t count, const int64_t *rows, const int64_t *cols,
                        double *out, double *den)
{
    if (count < 0 || (count > 0 && (rows == NULL || cols == NULL || out == NULL || den == NULL)))
        return ORACLE_EINVAL;
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_EINVAL;
    if (count == 0)
        return ORACLE_OK;
    if (M == 0 || N == 0)
        return ORACLE_EINVAL; /* there is no entry to sample */
    if ((K > 0 && (A == NULL || B == NULL)) || (beta != 0.0 && Cin == NULL))
        return ORACLE_EINVAL;
    for (int64_t e = 0; e < count; ++e)
        if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N)
            return ORACLE_EINVAL;

    int64_t e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < count; ++e) {
        int64_t m = rows[e], n = cols[e];
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = load_elem(A, kind, m * K + k) * load_elem(B, kind, k * N + n);
            acc += p;
            mag += fabs(p);
        }
        double c_in = (beta != 0.0) ? (double)Cin[m * N + n] : 0.0;
        out[e] = alpha * acc + beta * c_in;
        den[e] = fabs(alpha) * mag + fabs(beta * c_in) + 1e-30;
    }
    return ORACLE_OK;
}

/* ---- exported entry points (plain C ABI, host pointers only) ---- */

int oracle_gemm_f32(int64_t M, int64_t N, int64_t K, double alpha, double beta,
                    const float *A, const float *B, const float *Cin,
                    double *Cref, double *den)
{
    return gemm_full(M, N, K, alpha, beta, A, B, ELEM_F32, Cin, Cref, den);
}

int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K, double alpha, double beta,
                     const uint16_t *A, const uint16_t *B, const float *Cin,
                     double *Cref, double *den)
{
    return gemm_full(M, N, K, alpha, beta, A, B, ELEM_BF16, Cin, Cref, den);
}

int oracle_gemm_f32_entries(int64_t M, int64_t N, int64_t K, double alpha, double beta,
                            const float *A, const float *B, const float *Cin,
                            int64_t count, const int64_t *rows, const int64_t *cols,
                            double *out, double *den)
{
    return gemm_entries(M, N, K, alpha, beta, A, B, ELEM_F32, Cin, count, rows, cols, out, den);
}

int oracle_gemm_bf16_entries(int64_t M, int64_t N, int64_t K, double alpha, double beta,
                             const uint16_t *A, const uint16_t *B, const float *Cin,
                             int64_t count, const int64_t *rows, const int64_t *cols,
                             double *out, double *den)
{
    return gemm_entries(M, N, K, alpha, beta, A, B, ELEM_BF16, Cin, count, rows, cols, out, den);
}

/*
 * 8-bit floating-point inputs (the "smaller dtype raises the arithmetic
 * intensity" step of page "Where kernel performance comes from", section on
 * GEMM: 1-byte operands halve the bytes per multiply-add of bf16).  Two
 * formats, decoded exactly to double from their definitions:
 *   fmt 0, E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 *          0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinity;
 *   fmt 1, E5M2: sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent
 *          0 is subnormal (m/4 * 2^-14); exponent 31 is infinity (m = 0) or
 *          NaN.
 * The GEMM takes B stored N x K (row n holds column n of the product's
 * right operand, K contiguous) and per-tensor scales:
 *   C_ref[m][n] = alpha * sa * sb * sum_k A[m][k] * B[n][k] + beta * C_in[m][n]
 * with den = |alpha sa sb| * sum_k |A[m][k] B[n][k]| + |beta C_in| + 1e-30.
 */
static double fp8_value(uint8_t b, int fmt)
{
    const int s = b >> 7;
    double v;
    if (fmt == 0) {
        const int e = (b >> 3) & 15, m = b & 7;
        if (e == 15 && m == 7)
            return NAN;
        v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    } else {
        const int e = (b >> 2) & 31, m = b & 3;
        if (e == 31)
            return m == 0 ? (s ? -INFINITY : INFINITY) : NAN;
        v = e == 0 ? ldexp(m / 4.0, -14) : ldexp(1.0 + m / 4.0, e - 15);
    }
    return s ? -v : v;
}

int oracle_fp8_decode(int64_t n, const uint8_t *bytes, int fmt, double *out)
{
    if (n < 0 || (fmt != 0 && fmt != 1) || (n > 0 && (bytes == NULL || out == NULL)))
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        out[i] = fp8_value(bytes[i], fmt);
    return ORACLE_OK;
}

int oracle_gemm_fp8(int64_t M, int64_t N, int64_t K, double alpha, double beta, double sa,
                    double sb, int fmt, const uint8_t *A, const uint8_t *B, const float *Cin,
                    double *Cref, double *den)
{
    if (fmt != 0 && fmt != 1)
        return ORACLE_EINVAL;
    int rc = check_args(M, N, K, beta, A, B, Cin, Cref, den);
    if (rc != ORACLE_OK || M == 0 || N == 0)
        return rc;
    const double scale = alpha * sa * sb;
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = fp8_value(A[m * K + k], fmt) * fp8_value(B[n * K + k], fmt);
                acc += p;
                mag += fabs(p);
            }
            double c_in = (beta != 0.0) ? (double)Cin[m * N + n] : 0.0;
            Cref[m * N + n] = scale * acc + beta * c_in;
            den[m * N + n] = fabs(scale) * mag + fabs(beta * c_in) + 1e-30;
        }
    }
    return ORACLE_OK;
}

/*
 * Fused Linear-layer epilogue on a GEMM result.
 *
 * A Linear layer computes Y = XW + b (page "From model computation to GPU
 * execution", section 1.1), and an elementwise function such as GELU is the
 * typical consumer of its output (page "Where kernel performance comes
 * from", sections on elementwise kernels and on fusing a GEMM with its
 * elementwise epilogue).  Given z = alpha * A * B + beta * C_in from the
 * functions above, this computes
 *
 *     y = act(z + bias[n])
 *
 * in fp64, with bias an fp32 vector over the N output columns (NULL: no
 * bias) and act one of
 *
 *     0 identity   y = x
 *     1 ReLU       y = 0 for x < 0, else x   (NaN stays NaN)
 *     2 GELU       y = x * Phi(x) = x / 2 * erfc(-x / sqrt(2))
 *     3 SiLU       y = x / (1 + exp(-x))
 *
 * Entry e is column cols[e] (cols == NULL: column e % N, a full row-major
 * matrix).  The returned denominator is den_out[e] = slope * (den[e] +
 * |bias[n]|): an error e_z in z moves y by at most slope * e_z, where slope
 * bounds |act'| (1 for identity and ReLU; GELU' peaks at x = sqrt(2) at
 * 1.1289, SiLU' near x = 2.40 at 1.0998; 1.13 and 1.10 are used), so the
 * parity test |y_gpu - y| / den_out <= tol keeps the meaning it has for
 * plain GEMM.
 */
static double act_fn(int act, double x)
{
    switch (act) {
    case 1:
        return x < 0.0 ? 0.0 : x;
    case 2:
        return 0.5 * x * erfc(-x / sqrt(2.0)); /* Phi(x) without the 1 + erf cancellation */
    case 3:
        return x / (1.0 + exp(-x));
    default:
        return x;
    }
}

static double act_slope(int act)
{
    return act == 2 ? 1.13 : act == 3 ? 1.10 : 1.0;
}

int oracle_epilogue(int64_t count, int64_t N, const int64_t *cols, const double *z,
                    const double *den, const float *bias, int act, double *y, double *den_out)
{
    if (count < 0 || N < 0 || act < 0 || act > 3)
        return ORACLE_EINVAL;
    if (count == 0)
        return ORACLE_OK;
    if (N == 0 || z == NULL || den == NULL || y == NULL || den_out == NULL)
        return ORACLE_EINVAL;
    if (cols != NULL)
        for (int64_t e = 0; e < count; ++e)
            if (cols[e] < 0 || cols[e] >= N)
                return ORACLE_EINVAL;
    const double slope = act_slope(act);
    int64_t e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < count; ++e) {
        int64_t n = cols != NULL ? cols[e] : e % N;
        double b = bias != NULL ? (double)bias[n] : 0.0;
        y[e] = act_fn(act, z[e] + b);
        den_out[e] = slope * (den[e] + fabs(b));
    }
    return ORACLE_OK;
}

/*
 * Sum of a float32 vector: the memory-bound case study of page "Memory
 * hierarchy and cost table", section 4.7 (summing 100 million floats).
 * fp64, ascending index order; beside the sum, the sum of magnitudes
 * sum |x[i]| that scales the parity tolerance.  n == 0 gives 0 and 0.
 */
int oracle_sum_f32(int64_t n, const float *x, double *sum, double *abs_sum)
{
    if (n < 0 || sum == NULL || abs_sum == NULL || (n > 0 && x == NULL))
        return ORACLE_EINVAL;
    double s = 0.0, a = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        s += (double)x[i];
        a += fabs((double)x[i]);
    }
    *sum = s;
    *abs_sum = a;
    return ORACLE_OK;
}

/* Number of OpenMP threads a parallel region of this library would use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads later calls use (n >= 1); timing only,
 * the results do not depend on it (each output is summed by one thread in
 * ascending k). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
