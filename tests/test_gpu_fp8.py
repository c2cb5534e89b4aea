"""GPU parity of the 8-bit float GEMM (E4M3 and E5M2, B stored N x K, fp32
C) through the C ABI, against the oracle: both matrix-core kernels (the
128-deep K step one the library picks, and the 64-deep one
MGEMM_FP8_KERNEL selects: full K steps and a K tail, ragged M and N,
per-tensor scales, beta, split last rounds), the
one-thread-per-output fallback (K not a multiple of 16, unaligned operands),
K = 0, exact on integer inputs, within a tolerance derived from each
kernel's fp32 rounding chain (fp8_tol) on random inputs and on every finite
code (subnormals and the largest values included), and at the benchmarked
sizes over the whole output (E4M3) or 512 of its rows (E5M2)."""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import log
from roofline_driven_optimisation_amd import binding
from roofline_driven_optimisation_amd.inputs import _fp8_table, f32_to_fp8_bits

pytestmark = pytest.mark.gpu

FMTS = [0, 1]
FMT_ID = ["e4m3", "e5m2"]
KERNELS = ["fp8_q4_256x256x128", "fp8_q4_256x256x64"]  # the first is the default


@pytest.fixture(params=KERNELS)
def kernel(request, monkeypatch):
    """The matrix-core kernel under test (the 64-deep one by MGEMM_FP8_KERNEL)."""
    if request.param == KERNELS[0]:
        monkeypatch.delenv("MGEMM_FP8_KERNEL", raising=False)
    else:
        monkeypatch.setenv("MGEMM_FP8_KERNEL", request.param)
    return request.param


def expected(M, N, K, offset, kernel):
    """The kernel name gemm_fp8 reports: the one-thread-per-output kernel
    for K % 16 != 0 or unaligned operands, else the matrix-core kernel,
    with its last round split over K when that round is at most half full
    on 256 CUs and K has at least 8 of the kernel's steps (pairs on one XCD
    when the split tiles are a multiple of 8)."""
    if K % 16 or offset:
        return "naive_fp8"
    tiles = -(-M // 256) * -(-N // 256)
    r = tiles % 256
    steps = -(-K // int(kernel.rsplit("x", 1)[1]))
    if r and 2 * r <= 256 and steps >= 8:
        return kernel + ("_splitk_xcd" if r % 8 == 0 else "_splitk")
    return kernel

def fp8_tol(K, kernel):
    """Bound on max |C - C_ref| / den for the 8-bit float GEMM, from the
    arithmetic of each kernel.  Every E4M3 or E5M2 value and every product
    of two is exact in fp32 (at most 4 + 4 significant bits, exponents well
    inside fp32's range), so errors come only from how the products are
    summed:
      * matrix-core kernel: its instruction (v_mfma_scale_f32_32x32x64_
        f8f6f4) adds each group of 8 consecutive products in an adder
        aligned to the group's largest product and drops every other
        product's bits below 2^-13 of that product's leading bit
        (test_fp8_instruction_grouping pins this through gemm_fp8), so a
        group loses less than 7 * 2^-13 of its largest |product|, hence
        of its sum of |products|; the group sums, the accumulator, a split
        partner's partial, alpha and beta then go through at most
        8 ceil(K / 64) + 3 fp32 roundings, each under 2^-23 of a magnitude
        that never exceeds den;
      * one-thread-per-output kernel: K fp32 additions, then the folded
        scale, alpha and beta, each under 2^-24 of den.
    Rounding C (or any intermediate) to a 16-bit type would add up to 2^-9
    of |C|, which the positive-operand test, where |C| = den, catches."""
    if kernel.startswith("fp8_q4"):
        return 7 * 2.0 ** -13 + (8 * -(-K // 64) + 3) * 2.0 ** -23
    return 1.01 * (K + 3) * 2.0 ** -24


def draw(M, N, K, fmt, dist, seed):
    rng = np.random.default_rng(seed)
    if dist == "int":
        a = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
        b = rng.integers(-4, 5, size=(N, K)).astype(np.float32)
    elif dist == "codes":  # every finite code, uniformly
        _, codes = _fp8_table(fmt)
        return (rng.choice(codes, size=(M, K)).astype(np.uint8),
                rng.choice(codes, size=(N, K)).astype(np.uint8), rng)
    else:
        a = rng.standard_normal((M, K)).astype(np.float32)
        b = (rng.standard_normal((N, K)) * 0.5).astype(np.float32)
    return f32_to_fp8_bits(a, fmt), f32_to_fp8_bits(b, fmt), rng


def run(A, B, C, alpha, beta, sa, sb, fmt, offset=0):
    """C on the GPU; ``offset`` > 0 places A and B that many bytes past a
    16-byte boundary."""
    import torch
    M, K = A.shape
    N = B.shape[0]

    def dev(x):
        buf = torch.zeros(x.size + offset, dtype=torch.uint8, device="cuda")
        t = buf[offset:].view(x.shape)
        t.copy_(torch.from_numpy(x))
        return t

    At, Bt = dev(A), dev(B)
    Ct = (torch.from_numpy(C).cuda() if C is not None
          else torch.full((M, N), float("nan"), device="cuda"))
    log("  gpu fp8 fmt=%d %dx%dx%d alpha=%g beta=%g sa=%g sb=%g offset=%d" % (
        fmt, M, N, K, alpha, beta, sa, sb, offset))
    binding.gemm_fp8(At, Bt, Ct, alpha, beta, sa, sb, fmt)
    name = binding.last_kernel()
    torch.cuda.synchronize()
    return Ct.cpu().numpy(), name


CASES = [  # (M, N, K, offset)
    (256, 256, 64, 0),
    (300, 520, 256, 0),
    (300, 520, 144, 0),      # K tail of 16 (64-deep), of 16 after one step (128-deep)
    (520, 300, 1072, 0),     # K tail of 48, split pairs
    (37, 600, 16, 0),        # one partial K step
    (1, 1000, 512, 0),       # split by the 64-deep kernel, 4 steps for the 128-deep
    (1024, 512, 1024, 0),    # 8 split tiles: pairs on one XCD
    (1040, 520, 1104, 0),    # 15 split tiles, K tail of 16 (64-deep) or 80 (128-deep)
    (300, 520, 1936, 0),     # 16 steps of 128 less a 16-deep tail
    (70, 90, 60, 0),         # K % 16 != 0
    (70, 90, 64, 1),         # unaligned A and B
]


def ids(c):
    return "%dx%dx%d%s" % (c[0], c[1], c[2], "_off" if c[3] else "")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID)
@pytest.mark.parametrize("case", CASES, ids=ids)
def test_fp8_exact_integers(case, fmt, kernel):
    M, N, K, offset = case
    want = expected(M, N, K, offset, kernel)
    A, B, rng = draw(M, N, K, fmt, "int", seed=M + N + K)
    C = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    got, name = run(A, B, C, 1.0, 0.5, 1.0, 2.0, fmt, offset)
    assert name == want, name
    ref, _ = oracle.gemm_fp8(A, B, C, 1.0, 0.5, 1.0, 2.0, fmt)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID)
@pytest.mark.parametrize("case", CASES, ids=ids)
def test_fp8_random(case, fmt, kernel):
    M, N, K, offset = case
    want = expected(M, N, K, offset, kernel)
    A, B, _ = draw(M, N, K, fmt, "n", seed=7 + K)
    got, name = run(A, B, None, 1.25, 0.0, 0.5, 0.125, fmt, offset)
    assert name == want, name
    ref, den = oracle.gemm_fp8(A, B, None, 1.25, 0.0, 0.5, 0.125, fmt)
    err = oracle.parity_error(got, ref, den)
    log("  fp8 parity err=%.3e tol=%.2e" % (err, fp8_tol(K, name)))
    assert err <= fp8_tol(K, name)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID)
@pytest.mark.parametrize("offset", [0, 1], ids=["mfma", "naive"])
def test_fp8_every_finite_code(fmt, offset, kernel):
    """Operands drawn from every finite code of the format: subnormals,
    both zeros' neighbours and the largest magnitudes (448 and 57344)."""
    M, N, K = 264, 288, 320
    A, B, _ = draw(M, N, K, fmt, "codes", seed=11 + fmt)
    got, name = run(A, B, None, 1.0, 0.0, 1.0, 1.0, fmt, offset)
    assert name == ("naive_fp8" if offset else kernel), name
    ref, den = oracle.gemm_fp8(A, B, None, 1.0, 0.0, 1.0, 1.0, fmt)
    err = oracle.parity_error(got, ref, den)
    log("  fp8 all-codes err=%.3e tol=%.2e" % (err, fp8_tol(K, name)))
    assert err <= fp8_tol(K, name)


@pytest.mark.parametrize("shape", [(520, 300, 1072), (1024, 512, 1024)], ids=["pairs", "xcd"])
def test_fp8_split_repeats(shape, kernel):
    """Split tiles exchange partials through flags with a fresh epoch per
    call: three calls in a row give the same bits, equal to the oracle on
    integers."""
    M, N, K = shape
    A, B, rng = draw(M, N, K, 0, "int", seed=21)
    C = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    ref, _ = oracle.gemm_fp8(A, B, C, 1.0, 0.5, 1.0, 1.0, 0)
    for _ in range(3):
        got, name = run(A, B, C, 1.0, 0.5, 1.0, 1.0, 0)
        assert name == expected(M, N, K, 0, kernel) and "splitk" in name, name
        assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID)
def test_fp8_instruction_grouping(fmt, kernel):
    """The summation the matrix-core kernel's tolerance rests on, seen
    through gemm_fp8 on one output (M = N = 1, K = 64: one instruction; B
    stored N x K, so column 0 of B is its row 0): with a product 1 at k =
    0, a product 2^-13 at k = 1 survives, 2^-14 is dropped; at k = 8 (the
    next group of 8) 2^-14 survives; two 2^-14 products at k = 1 and 2 are
    each dropped, not summed first."""
    import torch
    from roofline_driven_optimisation_amd.inputs import f32_to_fp8_bits

    def one(pairs):
        a = np.zeros((1, 64), np.float32)
        b = np.zeros((1, 64), np.float32)
        for k, (x, y) in pairs.items():
            a[0, k], b[0, k] = x, y
        A, B = f32_to_fp8_bits(a, fmt), f32_to_fp8_bits(b, fmt)
        got, name = run(A, B, None, 1.0, 0.0, 1.0, 1.0, fmt)
        assert name == kernel, name
        return float(got[0, 0])

    h13, h14 = 2.0 ** -7, 2.0 ** -7  # 2^-13 = 2^-7 * 2^-6, 2^-14 = 2^-7 * 2^-7
    assert one({0: (1.0, 1.0), 1: (h13, 2.0 ** -6)}) == 1.0 + 2.0 ** -13
    assert one({0: (1.0, 1.0), 1: (h14, 2.0 ** -7)}) == 1.0
    assert one({0: (1.0, 1.0), 8: (h14, 2.0 ** -7)}) == 1.0 + 2.0 ** -14
    assert one({0: (1.0, 1.0), 1: (h14, 2.0 ** -7), 2: (h14, 2.0 ** -7)}) == 1.0


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID)
def test_fp8_positive_operands(fmt, kernel):
    """Positive operands make |C| equal to den, so the tolerance also
    bounds the error relative to C itself: an output rounded to a 16-bit
    type (2^-9 relative) would fail here."""
    M, N, K = 300, 520, 1024
    rng = np.random.default_rng(17 + fmt)
    A = f32_to_fp8_bits(np.abs(rng.standard_normal((M, K))).astype(np.float32), fmt)
    B = f32_to_fp8_bits(np.abs(rng.standard_normal((N, K)) * 0.5).astype(np.float32), fmt)
    got, name = run(A, B, None, 1.0, 0.0, 1.0, 1.0, fmt)
    assert name == expected(M, N, K, 0, kernel), name
    ref, den = oracle.gemm_fp8(A, B, None, 1.0, 0.0, 1.0, 1.0, fmt)
    err = oracle.parity_error(got, ref, den)
    log("  fp8 positive err=%.3e tol=%.2e (2^-9 = %.2e)" % (err, fp8_tol(K, name), 2.0 ** -9))
    assert err <= fp8_tol(K, name) < 2.0 ** -9 / 2


def test_fp8_k_zero():
    A = np.zeros((40, 0), np.uint8)
    B = np.zeros((72, 0), np.uint8)
    C = np.random.default_rng(1).integers(-4, 5, size=(40, 72)).astype(np.float32)
    got, name = run(A, B, C, 1.0, 0.5, 1.0, 1.0, 0)
    assert name == "scale_c", name
    assert np.array_equal(got, C * 0.5)


FULL = [(4096, 4096, 4096), (2048, 11008, 4096)]


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID)
@pytest.mark.parametrize("shape", FULL, ids=lambda c: "%dx%dx%d" % c[:3])
def test_fp8_full_size(shape, fmt):
    """The sizes the throughput is measured at (4096^3; 2048 x 11008 x 4096,
    whose third-full last round is split over K), with the kernel the
    library picks, against the oracle: the whole output for E4M3, the
    format the benchmark runs, and the 256 leading and 256 trailing rows
    for E5M2 (the oracle decodes every byte in its inner loop and takes
    over a minute per full product)."""
    M, N, K = shape
    want = expected(M, N, K, 0, KERNELS[0])
    A, B, rng = draw(M, N, K, fmt, "n", seed=5)
    got, name = run(A, B, None, 1.0, 0.0, 1.0, 1.0, fmt)
    assert name == want, name
    rows = np.arange(M) if fmt == 0 else np.r_[0:256, M - 256:M]
    ref, den = oracle.gemm_fp8(A[rows], B, None, 1.0, 0.0, 1.0, 1.0, fmt)
    err = oracle.parity_error(got[rows], ref, den)
    log("  fp8 %dx%dx%d, %d rows, err=%.3e tol=%.2e" % (M, N, K, len(rows), err,
                                                      fp8_tol(K, name)))
    assert err <= fp8_tol(K, name)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_ID)
@pytest.mark.parametrize("shape", FULL, ids=lambda c: "%dx%dx%d" % c[:3])
def test_fp8_full_size_integers(shape, fmt, kernel):
    """The benchmarked sizes with integer entries in [-4, 4] (exact in both
    formats; every product, group sum and partial sum is an integer below
    2^24, so exact in fp32 whatever the summation), on both kernels: the
    whole output must equal the product of the oracle's decoded operands,
    element for element, split tiles included."""
    M, N, K = shape
    want = expected(M, N, K, 0, kernel)
    A, B, _ = draw(M, N, K, fmt, "int", seed=8)
    got, name = run(A, B, None, 1.0, 0.0, 1.0, 1.0, fmt)
    assert name == want, name
    ref = oracle.fp8_decode(A, fmt) @ oracle.fp8_decode(B, fmt).T
    assert np.array_equal(got.astype(np.float64), ref)


def test_fp8_bad_arguments():
    import torch
    lib = binding.library()
    x = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    c = torch.zeros(4096, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.gemm_fp8(8, 8, 16, 1.0, 0.0, p(x), p(x), p(c), 1.0, 1.0, 2, s) == 1
    assert lib.gemm_fp8(-1, 8, 16, 1.0, 0.0, p(x), p(x), p(c), 1.0, 1.0, 0, s) == 1
    assert lib.gemm_fp8(8, 8, 16, 1.0, 0.0, None, p(x), p(c), 1.0, 1.0, 0, s) == 1
    assert lib.gemm_fp8(0, 8, 16, 1.0, 0.0, p(x), p(x), p(c), 1.0, 1.0, 0, s) == 0
    torch.cuda.synchronize()
