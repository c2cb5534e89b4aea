"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no GEMM arithmetic: it only draws random matrices and
rounds them to the storage formats.  Both sides of a parity check consume the
exact same bits produced here.

Recipe (the same for every workload): one ``numpy.random.default_rng(seed)``
generator draws A, then B, then C (only when beta != 0) in float64, which is
rounded to float32; bf16 operands are then rounded from float32 to bf16 with
round-to-nearest-even.  The workload table mirrors the shapes the pages use:
square 4096 and 4092 GEMMs (page "Naive GEMM and Roofline analysis",
sections 10.2.1 and 10.3.1) and LLaMA-7B projection / FFN shapes (d = 4096,
FFN 11008, vocabulary 32000; section 10.1 of the same page).  Trained weights
are not used anywhere: normal(0, 0.02) draws stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN stays NaN (quiet bit set).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fp8_table(fmt: int):
    """(finite values ascending, their bytes) of an 8-bit float format from
    its definition: fmt 0 E4M3 (bias 7, 3 mantissa bits, S.1111.111 NaN, no
    infinity), fmt 1 E5M2 (bias 15, 2 mantissa bits, exponent 31 inf/NaN)."""
    vals, codes = [], []
    for b in range(256):
        s = -1.0 if b & 0x80 else 1.0
        if fmt == 0:
            e, m = (b >> 3) & 15, b & 7
            if e == 15 and m == 7:
                continue
            v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        else:
            e, m = (b >> 2) & 31, b & 3
            if e == 31:
                continue
            v = (m / 4.0) * 2.0 ** -14 if e == 0 else (1 + m / 4.0) * 2.0 ** (e - 15)
        if v == 0.0 and s < 0:
            continue  # one zero: +0
        vals.append(s * v)
        codes.append(b)
    order = np.argsort(vals, kind="stable")
    return np.array(vals)[order], np.array(codes, dtype=np.uint8)[order]


def f32_to_fp8_bits(x: np.ndarray, fmt: int = 0) -> np.ndarray:
    """Round float32 values to an 8-bit float format (nearest, ties to the
    code with an even last mantissa bit; beyond the largest finite value,
    saturate to it).  Returns the bytes as uint8."""
    vals, codes = _fp8_table(fmt)
    x = np.asarray(x, dtype=np.float64)
    flat = np.clip(x.reshape(-1), vals[0], vals[-1])
    hi = np.clip(np.searchsorted(vals, flat), 1, len(vals) - 1)
    lo = hi - 1
    dlo, dhi = flat - vals[lo], vals[hi] - flat
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((codes[hi] & 1) == 0))
    out = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    return out.reshape(x.shape)


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    """One float32 matrix from a distribution spec.

    ``dist`` is one of ``"u"`` (uniform[-1, 1]), ``"n:<std>"`` (normal with
    mean 0 and that standard deviation), ``"i:<r>"`` (integers uniform in
    [-r, r], exact in bf16 and fp32 for r <= 256) or ``"ones"``.
    """
    if dist == "u":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist.startswith("n:"):
        std = float(dist[2:])
        return (rng.standard_normal(size=shape) * std).astype(np.float32)
    if dist.startswith("i:"):
        r = int(dist[2:])
        return rng.integers(-r, r + 1, size=shape).astype(np.float32)
    if dist == "ones":
        return np.ones(shape, dtype=np.float32)
    raise ValueError("unknown distribution %r" % dist)


@dataclass
class Case:
    """One GEMM problem instance with host operands.

    For ``dtype == "bf16"`` A and B are uint16 bf16 bit patterns; for
    ``"f32"`` they are float32.  C is float32, or None when beta == 0 (the
    GEMM then never reads C).
    """

    name: str
    M: int
    N: int
    K: int
    dtype: str
    alpha: float
    beta: float
    A: np.ndarray
    B: np.ndarray
    C: Optional[np.ndarray]
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"


def make_case(M: int, N: int, K: int, dtype: str = "f32", alpha: float = 1.0,
              beta: float = 0.0, dist_a: str = "u", dist_b: str = "u",
              dist_c: str = "u", seed: int = 0, name: str = "") -> Case:
    """Draw A (M x K), then B (K x N), then C (M x N, only if beta != 0)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    rng = np.random.default_rng(seed)
    A = _draw(rng, (M, K), dist_a)
    B = _draw(rng, (K, N), dist_b)
    C = _draw(rng, (M, N), dist_c) if beta != 0.0 else None
    if dtype == "bf16":
        A = f32_to_bf16_bits(A)
        B = f32_to_bf16_bits(B)
    return Case(name or "%s_%dx%dx%d" % (dtype, M, N, K), M, N, K, dtype,
                float(alpha), float(beta), A, B, C, seed)


def make_bias(N: int, dist: str = "n:0.5", seed: int = 0) -> np.ndarray:
    """A seeded float32 bias vector over N output columns (its own generator,
    seeded apart from the operands')."""
    return _draw(np.random.default_rng([seed, 0xB1A5]), (N,), dist)


@dataclass(frozen=True)
class Workload:
    """A named shape with its distributions, alpha and beta."""

    name: str
    M: int
    N: int
    K: int
    dtype: str
    alpha: float
    beta: float
    dist_a: str
    dist_b: str
    dist_c: str = "u"
    group: str = ""

    def case(self, seed: int = 0) -> Case:
        return make_case(self.M, self.N, self.K, self.dtype, self.alpha, self.beta,
                         self.dist_a, self.dist_b, self.dist_c, seed, self.name)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _bf16_std_for(K: int) -> str:
    return "n:%r" % float(1.0 / np.sqrt(K))


# The five workload groups.  Seeds are 0 for every shape.
WORKLOADS = [
    # square fp32, small enough for the full-matrix oracle in well under a second
    Workload("f32_256", 256, 256, 256, "f32", 1.0, 0.0, "u", "u", group="small"),
    # square fp32 at 4096 and at 4092 (edges that are not tile multiples)
    Workload("f32_4096", 4096, 4096, 4096, "f32", 1.5, 0.5, "u", "u", "u", group="square_f32"),
    Workload("f32_4092", 4092, 4092, 4092, "f32", 1.5, 0.5, "u", "u", "u", group="square_f32"),
    # square bf16 inputs, fp32 accumulate and output
    Workload("bf16_4096", 4096, 4096, 4096, "bf16", 1.0, 0.0, _bf16_std_for(4096),
             _bf16_std_for(4096), group="square_bf16"),
    # LLaMA-7B prefill projections: 2048 tokens
    Workload("prefill_qkv", 2048, 12288, 4096, "bf16", 1.0, 0.0, "n:1.0", "n:0.02", group="prefill"),
    Workload("prefill_o", 2048, 4096, 4096, "bf16", 1.0, 0.0, "n:1.0", "n:0.02", group="prefill"),
    Workload("prefill_gate_up", 2048, 11008, 4096, "bf16", 1.0, 0.0, "n:1.0", "n:0.02", group="prefill"),
    Workload("prefill_down", 2048, 4096, 11008, "bf16", 1.0, 0.0, "n:1.0", "n:0.02", group="prefill"),
]
for _m in (1, 8, 16):
    WORKLOADS.append(Workload("decode_up_m%d" % _m, _m, 11008, 4096, "bf16", 1.0, 0.0,
                              "n:1.0", "n:0.02", group="decode"))
for _m in (1, 8, 16):
    WORKLOADS.append(Workload("decode_down_m%d" % _m, _m, 4096, 11008, "bf16", 1.0, 0.0,
                              "n:1.0", "n:0.02", group="decode"))
WORKLOADS.append(Workload("decode_lm_head", 1, 32000, 4096, "bf16", 1.0, 0.0,
                          "n:1.0", "n:0.02", group="decode"))

WORKLOADS_BY_NAME = {w.name: w for w in WORKLOADS}


def workload(name: str) -> Workload:
    return WORKLOADS_BY_NAME[name]
