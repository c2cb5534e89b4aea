"""CPU oracle for C = alpha*A*B + beta*C, used as test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and the
two share no code: this module wraps ``oracle_gemm.c`` (plain C, fp64
accumulation, built with gcc) through ctypes.

The definition it follows is the GEMM formula of page "Naive GEMM and
Roofline analysis", section 10.1, with the row-major indexing of that page's
naive kernel (section 10.2).  Every function returns the fp64 result together
with the parity denominator ``|alpha| * sum_k |A*B| + |beta*C_in| + 1e-30``.
The optional fused epilogue (bias over the N columns, then an activation)
follows the Linear layer Y = XW + b of page "From model computation to GPU
execution", section 1.1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle_gemm.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")


def compile_library(src: str, out: str) -> str:
    """gcc -O2 -fopenmp: plain IEEE fp64 (no -ffast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Werror", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle_gemm.c into oracle/liboracle.so."""
    if force or not os.path.exists(LIB_PATH):
        compile_library(SOURCE, LIB_PATH)
    return LIB_PATH


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, f64, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        for name in ("oracle_gemm_f32", "oracle_gemm_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [i64, i64, i64, f64, f64, vp, vp, vp, vp, vp]
            fn.restype = ctypes.c_int
        for name in ("oracle_gemm_f32_entries", "oracle_gemm_bf16_entries"):
            fn = getattr(lib, name)
            fn.argtypes = [i64, i64, i64, f64, f64, vp, vp, vp, i64, vp, vp, vp, vp]
            fn.restype = ctypes.c_int
        lib.oracle_epilogue.argtypes = [i64, i64, vp, vp, vp, vp, ctypes.c_int, vp, vp]
        lib.oracle_epilogue.restype = ctypes.c_int
        lib.oracle_fp8_decode.argtypes = [i64, vp, ctypes.c_int, vp]
        lib.oracle_fp8_decode.restype = ctypes.c_int
        lib.oracle_gemm_fp8.argtypes = [i64, i64, i64, f64, f64, f64, f64, ctypes.c_int,
                                        vp, vp, vp, vp, vp]
        lib.oracle_gemm_fp8.restype = ctypes.c_int
        lib.oracle_sum_f32.argtypes = [i64, vp, vp, vp]
        lib.oracle_sum_f32.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        self.lib = lib
        self.path = path

    @staticmethod
    def _operands(A, B, C, beta, bf16):
        want = np.uint16 if bf16 else np.float32
        A = np.ascontiguousarray(A)
        B = np.ascontiguousarray(B)
        if A.dtype != want or B.dtype != want:
            raise TypeError("A and B must be %s arrays" % np.dtype(want).name)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
            raise ValueError("shapes do not chain: %s x %s" % (A.shape, B.shape))
        M, K = A.shape
        N = B.shape[1]
        if beta != 0.0:
            if C is None:
                raise ValueError("beta != 0 needs C_in")
            C = np.ascontiguousarray(C, dtype=np.float32)
            if C.shape != (M, N):
                raise ValueError("C_in must be %dx%d" % (M, N))
        else:
            C = None  # never read when beta == 0
        return A, B, C, M, N, K

    def epilogue(self, z, den, bias=None, act=0, cols=None):
        """Fused Linear-layer epilogue y = act(z + bias[n]) on a GEMM result z
        (fp64, with its denominator den): returns (y, den_out), den_out being
        the activation's slope bound times (den + |bias[n]|).  ``cols`` gives
        each entry's column for sampled entries; None means z is a full
        row-major matrix whose last axis is N.  act: 0 identity, 1 ReLU,
        2 GELU (erf form), 3 SiLU."""
        z = np.ascontiguousarray(z, dtype=np.float64)
        den = np.ascontiguousarray(den, dtype=np.float64)
        if z.shape != den.shape:
            raise ValueError("z and den differ in shape")
        if cols is None:
            N = z.shape[-1] if z.ndim == 2 else 0
            if z.ndim != 2:
                raise ValueError("a full result must be 2-D")
        else:
            cols = np.ascontiguousarray(cols, dtype=np.int64)
            if cols.shape != z.shape or z.ndim != 1:
                raise ValueError("cols must match the sampled entries")
            N = None
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
            if bias.ndim != 1:
                raise ValueError("bias must be a vector")
            if N is None:
                N = bias.shape[0]
            elif bias.shape[0] != N:
                raise ValueError("bias must have N = %d entries" % N)
        if N is None:
            N = int(cols.max()) + 1 if cols.size else 1
        y = np.empty_like(z)
        den_out = np.empty_like(z)
        rc = self.lib.oracle_epilogue(z.size, N, _ptr(cols), _ptr(z), _ptr(den), _ptr(bias),
                                      int(act), _ptr(y), _ptr(den_out))
        if rc != 0:
            raise ValueError("oracle rejected the epilogue arguments (code %d)" % rc)
        return y, den_out

    def gemm(self, A, B, C=None, alpha=1.0, beta=0.0, bf16=False, bias=None, act=0):
        """Full fp64 reference: (C_ref, den), both float64 M x N arrays.

        ``bf16=True``: A and B are uint16 arrays of bf16 bit patterns,
        otherwise float32.  C is float32 and is read only when beta != 0.
        With ``bias`` (fp32, N entries) or ``act`` the result is the fused
        Linear-layer output act(alpha * A * B + beta * C + bias) and den the
        matching epilogue denominator (see ``epilogue``).
        """
        A, B, C, M, N, K = self._operands(A, B, C, beta, bf16)
        Cref = np.empty((M, N), dtype=np.float64)
        den = np.empty((M, N), dtype=np.float64)
        fn = self.lib.oracle_gemm_bf16 if bf16 else self.lib.oracle_gemm_f32
        rc = fn(M, N, K, float(alpha), float(beta), _ptr(A), _ptr(B), _ptr(C),
                _ptr(Cref), _ptr(den))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (code %d)" % rc)
        if bias is not None or act:
            return self.epilogue(Cref, den, bias, act)
        return Cref, den

    def gemm_entries(self, A, B, rows, cols, C=None, alpha=1.0, beta=0.0, bf16=False,
                     bias=None, act=0):
        """fp64 reference at the sampled positions (rows[e], cols[e]) only."""
        A, B, C, M, N, K = self._operands(A, B, C, beta, bf16)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape or rows.ndim != 1:
            raise ValueError("rows and cols must be 1-D and of equal length")
        out = np.empty(rows.shape[0], dtype=np.float64)
        den = np.empty(rows.shape[0], dtype=np.float64)
        fn = self.lib.oracle_gemm_bf16_entries if bf16 else self.lib.oracle_gemm_f32_entries
        rc = fn(M, N, K, float(alpha), float(beta), _ptr(A), _ptr(B), _ptr(C),
                rows.shape[0], _ptr(rows), _ptr(cols), _ptr(out), _ptr(den))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (code %d)" % rc)
        if bias is not None or act:
            if bias is not None and np.asarray(bias).shape != (N,):
                raise ValueError("bias must have N = %d entries" % N)
            return self.epilogue(out, den, bias, act, cols=cols)
        return out, den

    def gemm_batched(self, A, B, C=None, alpha=1.0, beta=0.0, bf16=False, trans_b=False):
        """Strided batched GEMM, item by item: A (batch, M, K), B (batch, K, N)
        or, with ``trans_b``, (batch, N, K) holding each item's B transposed;
        C (batch, M, N) or None.  Returns (C_ref, den) of shape (batch, M, N).
        This is the attention use of the GEMM: S = Q K^T and O = P V (page
        "From model computation to GPU execution", section 1.2), one GEMM per
        head (page "Naive GEMM and Roofline analysis", section 10.1), with K
        stored token-major (Seq_k x d), i.e. as B transposed.  One plain GEMM
        per item."""
        A = np.asarray(A)
        B = np.asarray(B)
        if A.ndim != 3 or B.ndim != 3 or A.shape[0] != B.shape[0]:
            raise ValueError("A and B must be (batch, rows, cols) with one batch size")
        outs, dens = [], []
        for b in range(A.shape[0]):
            Bb = np.ascontiguousarray(B[b].T) if trans_b else B[b]
            Cb = None if C is None else C[b]
            r, d = self.gemm(A[b], Bb, Cb, alpha, beta, bf16)
            outs.append(r)
            dens.append(d)
        M, N = A.shape[1], (B.shape[1] if trans_b else B.shape[2])
        if not outs:
            return np.zeros((0, M, N)), np.zeros((0, M, N))
        return np.stack(outs), np.stack(dens)

    def fp8_decode(self, b, fmt=0):
        """Exact values (float64) of 8-bit float bytes: fmt 0 E4M3, 1 E5M2."""
        b = np.ascontiguousarray(b, dtype=np.uint8)
        out = np.empty(b.shape, dtype=np.float64)
        rc = self.lib.oracle_fp8_decode(b.size, _ptr(b), int(fmt), _ptr(out))
        if rc != 0:
            raise ValueError("oracle rejected the decode arguments (code %d)" % rc)
        return out

    def gemm_fp8(self, A, B, C=None, alpha=1.0, beta=0.0, sa=1.0, sb=1.0, fmt=0):
        """fp64 reference of the 8-bit float GEMM: A (M x K) and B stored
        N x K as uint8 bytes, C fp32 (read when beta != 0):
        alpha sa sb A B^T + beta C.  Returns (C_ref, den)."""
        A = np.ascontiguousarray(A, dtype=np.uint8)
        B = np.ascontiguousarray(B, dtype=np.uint8)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
            raise ValueError("A is M x K and B is N x K")
        M, K = A.shape
        N = B.shape[0]
        if beta != 0.0:
            C = np.ascontiguousarray(C, dtype=np.float32)
            if C.shape != (M, N):
                raise ValueError("C_in must be %dx%d" % (M, N))
        else:
            C = None
        Cref = np.empty((M, N), dtype=np.float64)
        den = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_fp8(M, N, K, float(alpha), float(beta), float(sa), float(sb),
                                      int(fmt), _ptr(A), _ptr(B), _ptr(C), _ptr(Cref), _ptr(den))
        if rc != 0:
            raise ValueError("oracle rejected the fp8 arguments (code %d)" % rc)
        return Cref, den

    def sum_f32(self, x):
        """fp64 sum of a float32 vector and its sum of magnitudes (the
        reduction case study of page "Memory hierarchy and cost table",
        section 4.7): returns (sum, abs_sum)."""
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        out = np.zeros(2, dtype=np.float64)
        rc = self.lib.oracle_sum_f32(x.size, _ptr(x), out.ctypes.data_as(ctypes.c_void_p),
                                     ctypes.c_void_p(out.ctypes.data + 8))
        if rc != 0:
            raise ValueError("oracle rejected the sum arguments (code %d)" % rc)
        return float(out[0]), float(out[1])

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _default = Oracle(LIB_PATH)
    return _default


def gemm(A, B, C=None, alpha=1.0, beta=0.0, bf16=False, bias=None, act=0):
    return default().gemm(A, B, C, alpha, beta, bf16, bias, act)


def gemm_entries(A, B, rows, cols, C=None, alpha=1.0, beta=0.0, bf16=False, bias=None, act=0):
    return default().gemm_entries(A, B, rows, cols, C, alpha, beta, bf16, bias, act)


def epilogue(z, den, bias=None, act=0, cols=None):
    return default().epilogue(z, den, bias, act, cols)


def sum_f32(x):
    return default().sum_f32(x)


def fp8_decode(b, fmt=0):
    return default().fp8_decode(b, fmt)


def gemm_fp8(A, B, C=None, alpha=1.0, beta=0.0, sa=1.0, sb=1.0, fmt=0):
    return default().gemm_fp8(A, B, C, alpha, beta, sa, sb, fmt)


def gemm_batched(A, B, C=None, alpha=1.0, beta=0.0, bf16=False, trans_b=False):
    return default().gemm_batched(A, B, C, alpha, beta, bf16, trans_b)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use in this process."""
    return default().num_threads()


def set_num_threads(n: int) -> None:
    """Threads for later oracle calls (timing only; results do not change)."""
    default().set_num_threads(n)


def parity_error(c_gpu, c_ref, den) -> float:
    """max |c - c_ref| / den, NaN-propagating: any non-finite GPU value where
    the reference is finite counts as an infinite error."""
    c = np.asarray(c_gpu, dtype=np.float64)
    err = np.abs(c - c_ref) / den
    bad = ~np.isfinite(c) & np.isfinite(c_ref)
    if bad.any():
        return float("inf")
    if err.size == 0:
        return 0.0
    return float(np.max(err))
