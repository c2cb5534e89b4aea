"""Helpers for the GPU parity tests: move seeded cases to the device, run the
library through its C ABI, and compare against the CPU oracle."""
import numpy as np

import oracle
from oracle import parity_error
from roofline_driven_optimisation_amd import binding

# Parity tolerances on max |C - C_ref| / (|alpha| sum_k |A B| + |beta C| + 1e-30)
TOL = {"f32": 1e-5, "bf16": 4e-3}


def log(msg):
    print(msg, flush=True)


def to_device(case, c_fill=np.nan):
    """Device tensors for a Case.  With beta == 0 C starts as ``c_fill``
    (NaN by default) to prove that it is never read."""
    import torch
    if case.bf16:
        A = torch.from_numpy(case.A.view(np.int16)).view(torch.bfloat16).cuda()
        B = torch.from_numpy(case.B.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        A = torch.from_numpy(case.A).cuda()
        B = torch.from_numpy(case.B).cuda()
    if case.C is not None:
        C = torch.from_numpy(case.C).cuda()
    else:
        C = torch.full((case.M, case.N), float(c_fill), dtype=torch.float32, device="cuda")
    return A, B, C


def run(case, kernel="auto", stream=None, c_fill=np.nan):
    """Run one GEMM on the GPU; returns (C as float32 numpy, kernel name)."""
    import torch
    A, B, C = to_device(case, c_fill)
    log("  gpu %s %dx%dx%d %s alpha=%g beta=%g kernel=%s" % (
        case.name, case.M, case.N, case.K, case.dtype, case.alpha, case.beta, kernel))
    fn = {"auto": binding.gemm, "naive": (binding.gemm_naive_bf16 if case.bf16
                                          else binding.gemm_naive_f32)}[kernel]
    # the pure dispatch query names the kernel before the call launches it
    # (it assumes the null stream, which torch's default stream is)
    predicted = binding.kernel_name(case.dtype, case.M, case.N, case.K)
    fn(A, B, C, case.alpha, case.beta, stream=stream)
    name = binding.last_kernel()
    if kernel == "auto" and stream is None:
        assert predicted == name, "gemm_kernel_name %s, launched %s" % (predicted, name)
    torch.cuda.synchronize()
    return C.cpu().numpy(), name


def oracle_full(case):
    return oracle.gemm(case.A, case.B, case.C, case.alpha, case.beta, bf16=case.bf16)


def sample_positions(M, N, count, seed=0, tiles=(32, 128, 256)):
    """Seeded sample of output positions: random ones plus every corner,
    the last row and column, and both sides of tile boundaries."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, count))
    cols = list(rng.integers(0, N, count))
    edge_r = {0, M - 1}
    edge_c = {0, N - 1}
    for t in tiles:
        for b in range(t, max(M, N), t):
            if b < M:
                edge_r.update({b - 1, b})
            if b < N:
                edge_c.update({b - 1, b})
    edge_r = sorted(edge_r)
    edge_c = sorted(edge_c)
    for r in edge_r:
        rows.append(r)
        cols.append(int(rng.integers(0, N)))
    for c in edge_c:
        rows.append(int(rng.integers(0, M)))
        cols.append(c)
    for r in (0, M - 1):
        for c in (0, N - 1):
            rows.append(r)
            cols.append(c)
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def check_full(case, C_gpu, tol=None):
    Cref, den = oracle_full(case)
    err = parity_error(C_gpu, Cref, den)
    tol = TOL[case.dtype] if tol is None else tol
    log("  parity(full) %s err=%.3e tol=%.1e" % (case.name, err, tol))
    assert err <= tol, "%s: parity error %.3e > %.1e" % (case.name, err, tol)
    return err


def check_sampled(case, C_gpu, count=2048, seed=0):
    rows, cols = sample_positions(case.M, case.N, count, seed)
    ref, den = oracle.gemm_entries(case.A, case.B, rows, cols, case.C, case.alpha, case.beta,
                                   bf16=case.bf16)
    err = parity_error(C_gpu[rows, cols], ref, den)
    log("  parity(sampled %d) %s err=%.3e" % (len(rows), case.name, err))
    assert err <= TOL[case.dtype], "%s: parity error %.3e" % (case.name, err)
    return err


def operands_f64(case):
    from roofline_driven_optimisation_amd.inputs import bf16_bits_to_f32
    if case.bf16:
        return (bf16_bits_to_f32(case.A).astype(np.float64),
                bf16_bits_to_f32(case.B).astype(np.float64))
    return case.A.astype(np.float64), case.B.astype(np.float64)


def check_row_checksums(case, C_gpu):
    """A property that holds at any size: for every row m,
    sum_n C[m][n] = alpha * sum_k A[m][k] (sum_n B[k][n]) + beta * sum_n C_in[m][n],
    within the tolerance applied to the summed denominators
    |alpha| sum_k |A[m][k]| sum_n |B[k][n]| + |beta| sum_n |C_in[m][n]|."""
    A, B = operands_f64(case)
    lhs = C_gpu.astype(np.float64).sum(axis=1)
    rhs = case.alpha * (A @ B.sum(axis=1))
    bound = abs(case.alpha) * (np.abs(A) @ np.abs(B).sum(axis=1))
    if case.beta != 0.0:
        Cin = case.C.astype(np.float64)
        rhs = rhs + case.beta * Cin.sum(axis=1)
        bound = bound + abs(case.beta) * np.abs(Cin).sum(axis=1)
    err = float(np.max(np.abs(lhs - rhs) / (bound + 1e-30)))
    log("  row checksums %s err=%.3e" % (case.name, err))
    assert np.all(np.isfinite(C_gpu))
    assert err <= TOL[case.dtype]
