"""Benchmark of the GEMM library on one MI355X; prints ONE JSON line.

A step is one call of the hot path on the headline workload, bf16-input /
fp32-accumulate GEMM at M = N = K = 4096 (alpha = 1, beta = 0), with inputs
already resident in HBM.  ``value`` is that GEMM's throughput in TFLOP/s over
exactly ``--steps`` timed steps (after ``--warmup`` untimed ones), bracketed
by device synchronisations.  The same line carries:

* ``roofline``: the dominant kernel's achieved TFLOP/s (2*M*N*K per launch
  over the average launch time from HIP events recorded on the launch
  stream) against the bf16 MFMA peak, plus HBM traffic from rocprofv3
  counters when a counter summary for the current kernel source exists;
* ``also``: the other workloads (fp32 4096^3 and 4092^3 with alpha 1.5 and
  beta 0.5, LLaMA-7B prefill projections, decode-shaped GEMMs, the fused
  bias + activation epilogue, the 10^8-float vector sum, attention's batched
  QK^T and PV, 8-bit float GEMMs) with TFLOP/s, algorithmic GB/s and their
  own roofline fraction;
* ``ladder``: the one-thread-per-output kernel against the tiled one on
  fp32 4092^3, the first and last rungs of the optimisation ladder;
* ``page_context``: the figures the pages quote for other machines;
* ``cpu_baseline``: the CPU oracle, as it stands, timed (rank 0, N = 1 only)
  on the whole headline GEMM and on sampled rows of every other workload,
  with a per-configuration list and configuration 1 also single-threaded;
* ``parity`` (for the headline, and in each ``also`` entry): after each
  workload's timed loop, one more launch keeps sampled rows of its output,
  which the oracle leg above compares with its own rows (max |C - C_ref| /
  den against the workload's tolerance).

``--sustain SECONDS`` instead launches a workload back to back and samples
the GFX clock and board power with amd-smi (the GEMM runs at the power limit).

Every timed launch cycles through several copies of the operands whose total
exceeds twice the 256 MB last-level cache, so each launch streams from HBM.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from roofline_driven_optimisation_amd import roofline as rl  # noqa: E402
from roofline_driven_optimisation_amd.inputs import workload  # noqa: E402

HEADLINE = "bf16_4096"
SECONDARY = ["f32_4096", "f32_4092", "prefill_qkv", "prefill_o", "prefill_gate_up",
             "prefill_down", "decode_up_m1", "decode_up_m8", "decode_up_m16",
             "decode_down_m1", "decode_down_m8", "decode_down_m16", "decode_lm_head",
             "prefill_gate_up+bias_gelu", "decode_up_m1+bias_silu", "sum_1e8",
             "attn_qk", "attn_pv", "fp8_4096", "fp8_prefill_gate_up"]
# "<workload>+bias_<act>": the workload through the fused Linear-layer
# epilogue, C = act(A*B + bias) with a normal(0, 0.5) bias over the columns
ACTIVATIONS = {"none": 0, "relu": 1, "gelu": 2, "silu": 3}
ROTATE_BYTES = 2 * 256 * 2 ** 20  # twice the MI355X Infinity Cache


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kernel_name: str) -> str:
    """Hash of the source file that defines a kernel family (to tell whether
    stored counter readings still describe the current code)."""
    from roofline_driven_optimisation_amd.profiling import source_hash
    return source_hash(kernel_name)


def stored_traffic(kernel_name: str, workload_name: str):
    """HBM bytes per launch from a committed counter summary, or None.

    The summary (profiles/counters_<kernel>_<workload>.md) states the source
    hash it was taken with and the calibrated FETCH/WRITE bytes per dispatch;
    a different hash means the kernel changed and the reading is stale.
    """
    path = os.path.join(ROOT, "profiles", "counters_%s_%s.md" % (kernel_name, workload_name))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(kernel_name):
        return None
    return float(m_bytes.group(1))


class Prepared:
    """Device copies of one workload's operands, rotated across launches."""

    def __init__(self, name: str, seed: int = 0):
        import torch
        from roofline_driven_optimisation_amd.inputs import make_bias
        base, _, epi = name.partition("+")
        self.name = name
        self.w = workload(base)
        self.epi = None
        if epi:
            if not epi.startswith("bias_") or epi[5:] not in ACTIVATIONS:
                raise ValueError("unknown epilogue %r" % epi)
            bias = torch.from_numpy(make_bias(self.w.N, "n:0.5", seed)).cuda()
            self.epi = (bias, ACTIVATIONS[epi[5:]])
        case = self.w.case(seed)
        self.case = case
        if case.bf16:
            A = torch.from_numpy(case.A.view(np.int16)).view(torch.bfloat16)
            B = torch.from_numpy(case.B.view(np.int16)).view(torch.bfloat16)
        else:
            A = torch.from_numpy(case.A)
            B = torch.from_numpy(case.B)
        C = (torch.from_numpy(case.C) if case.C is not None
             else torch.zeros(case.M, case.N, dtype=torch.float32))
        per_set = (A.numel() * A.element_size() + B.numel() * B.element_size()
                   + C.numel() * C.element_size())
        self.sets = max(1, -(-ROTATE_BYTES // per_set))
        A, B, C = A.cuda(), B.cuda(), C.cuda()
        self.bufs = [(A, B, C)] + [(A.clone(), B.clone(), C.clone()) for _ in range(self.sets - 1)]
        self.C0 = C.clone() if case.C is not None else None
        self.rf = rl.gemm_roofline(case.M, case.N, case.K, case.dtype, case.beta != 0.0,
                                   bias=self.epi is not None)

    def launch(self, i: int, naive: bool = False):
        from roofline_driven_optimisation_amd import binding
        A, B, C = self.bufs[i % self.sets]
        if naive:
            fn = binding.gemm_naive_bf16 if self.case.bf16 else binding.gemm_naive_f32
            fn(A, B, C, self.w.alpha, self.w.beta)
        elif self.epi is not None:
            fn = binding.gemm_bf16_bias_act if self.case.bf16 else binding.gemm_f32_bias_act
            fn(A, B, C, self.epi[0], self.epi[1], self.w.alpha, self.w.beta)
        else:
            binding.gemm(A, B, C, self.w.alpha, self.w.beta)

    def kernel_name(self) -> str:
        from roofline_driven_optimisation_amd import binding
        self.launch(0)
        return binding.last_kernel()

    # -- parity of a sampled block, outside the timed region --------------
    def rows_for(self, budget_flop):
        return sample_rows(self.w.M, self.w.N, self.w.K, budget_flop)

    def verify_launch(self, rows):
        """One more launch on operand set 0 (C restored first when beta !=
        0); returns the GPU output's `rows`."""
        import torch
        A, B, C = self.bufs[0]
        if self.C0 is not None:
            C.copy_(self.C0)
        self.launch(0)
        torch.cuda.synchronize()
        if self.epi is not None:
            self.bias_host = self.epi[0].cpu().numpy()
        return C[torch.from_numpy(rows).cuda()].cpu().numpy()

    def oracle_rows(self, rows):
        """(reference, denominator, FLOPs) of the oracle on `rows`."""
        import oracle
        c = self.case
        bias = act = None
        if self.epi is not None:
            bias, act = self.bias_host, self.epi[1]
        ref, den = oracle.gemm(c.A[rows], c.B, c.C[rows] if c.C is not None else None,
                               c.alpha, c.beta, bf16=c.bf16, bias=bias, act=act or 0)
        return ref, den, 2.0 * len(rows) * c.N * c.K

    def tolerance(self):
        tol = 4e-3 if self.case.bf16 else 1e-5
        if self.epi is not None:  # |act'| bounds how far an error moves the output
            tol *= {0: 1.0, 1: 1.0, 2: 1.13, 3: 1.10}[self.epi[1]]
        return tol


def sample_rows(M, N, K, budget_flop):
    """Output rows checked against the oracle: all of them when the budget
    allows (and always at M <= 16), else equal numbers of leading and
    trailing rows (the first and the last, possibly ragged, tile rows)."""
    per_row = 2.0 * N * K
    if M <= 16 or budget_flop == float("inf"):
        count = M
    else:
        count = int(min(M, max(2, budget_flop // per_row)))
    if count >= M:
        return np.arange(M, dtype=np.int64)
    half = max(1, count // 2)
    return np.concatenate([np.arange(half), np.arange(M - half, M)]).astype(np.int64)


class PreparedSum:
    """The vector-sum workload "sum_<n>": n float32 values ~ U[-1, 1] (seed
    0), rotated across copies like the GEMM operands; ``naive`` launches the
    one-element-per-thread first version."""

    def __init__(self, name: str, seed: int = 0):
        import torch
        self.name = name
        self.n = int(float(name.split("_", 1)[1]))
        x = np.random.default_rng(seed).uniform(-1.0, 1.0, self.n).astype(np.float32)
        self.sets = max(1, -(-ROTATE_BYTES // (4 * self.n)))
        xt = torch.from_numpy(x).cuda()
        self.bufs = [xt] + [xt.clone() for _ in range(self.sets - 1)]
        self.out = torch.zeros(1, dtype=torch.float32, device="cuda")
        self.rf = rl.sum_roofline(self.n)

    def launch(self, i: int, naive: bool = False):
        from roofline_driven_optimisation_amd import binding
        binding.reduce_sum_f32(self.bufs[i % self.sets], self.out, naive=naive)

    def rows_for(self, budget_flop):
        return None  # the whole vector

    def verify_launch(self, rows):
        import torch
        self.x_host = self.bufs[0].cpu().numpy()
        self.launch(0)
        torch.cuda.synchronize()
        return self.out.cpu().numpy()[:1]

    def oracle_rows(self, rows):
        import oracle
        s, a = oracle.sum_f32(self.x_host)
        return np.array([s]), np.array([a + 1e-30]), float(self.n)

    def tolerance(self):
        # at most n / 2^21 + 32 fp32 additions per element (80 at 10^8)
        return (self.n / 2.0 ** 21 + 32) * 2.0 ** -24

    def kernel_name(self) -> str:
        from roofline_driven_optimisation_amd import binding
        self.launch(0)
        return binding.last_kernel()


# attention GEMMs of one layer: 32 heads, 2048 tokens, head dimension 128
ATTENTION = {"attn_qk": (32, 2048, 2048, 128, True), "attn_pv": (32, 2048, 128, 2048, False)}


class PreparedBatched:
    """Strided batched bf16 GEMM: S = Q K^T (K stored token-major, so B is
    transposed) or O = P V, per head; Q, K, V ~ normal(0, 1) and P ~
    uniform[0, 1/64] rounded to bf16 (seed 0), rotated across copies."""

    def __init__(self, name: str, seed: int = 0):
        import torch
        from roofline_driven_optimisation_amd.inputs import f32_to_bf16_bits
        self.name = name
        self.batch, self.M, self.N, self.K, self.trans_b = ATTENTION[name]
        rng = np.random.default_rng(seed)
        b, M, N, K = self.batch, self.M, self.N, self.K
        if self.trans_b:
            a = rng.standard_normal((b, M, K)).astype(np.float32)
            bb = rng.standard_normal((b, N, K)).astype(np.float32)
        else:
            a = rng.uniform(0.0, 1.0 / 64, (b, M, K)).astype(np.float32)
            bb = rng.standard_normal((b, K, N)).astype(np.float32)
        A = torch.from_numpy(f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()
        B = torch.from_numpy(f32_to_bf16_bits(bb).view(np.int16)).view(torch.bfloat16).cuda()
        C = torch.zeros(b, M, N, dtype=torch.float32, device="cuda")
        per_set = 2 * (A.numel() + B.numel()) + 4 * C.numel()
        self.sets = max(1, -(-ROTATE_BYTES // per_set))
        self.bufs = [(A, B, C)] + [(A.clone(), B.clone(), C.clone()) for _ in range(self.sets - 1)]
        self.rf = rl.batched_gemm_roofline(b, M, N, K, "bf16")

    def launch(self, i: int, naive: bool = False):
        from roofline_driven_optimisation_amd import binding
        A, B, C = self.bufs[i % self.sets]
        binding.gemm_bf16_batched(A, B, C, 1.0, 0.0, trans_b=self.trans_b)

    def rows_for(self, budget_flop):  # rows of the first head
        return sample_rows(self.M, self.N, self.K, budget_flop)

    def verify_launch(self, rows):
        import torch
        A, B, C = self.bufs[0]
        self.launch(0)
        torch.cuda.synchronize()
        self.a0 = A[0].view(torch.int16).cpu().numpy().view(np.uint16)
        self.b0 = B[0].view(torch.int16).cpu().numpy().view(np.uint16)
        return C[0][torch.from_numpy(rows).cuda()].cpu().numpy()

    def oracle_rows(self, rows):
        import oracle
        b = np.ascontiguousarray(self.b0.T) if self.trans_b else self.b0
        ref, den = oracle.gemm(self.a0[rows], b, None, 1.0, 0.0, bf16=True)
        return ref, den, 2.0 * len(rows) * self.N * self.K

    def tolerance(self):
        return 4e-3

    def kernel_name(self) -> str:
        from roofline_driven_optimisation_amd import binding
        self.launch(0)
        return binding.last_kernel()


# 8-bit float GEMMs (E4M3 operands, B stored N x K, fp32 C, beta = 0):
# name -> (M, N, K)
FP8 = {"fp8_4096": (4096, 4096, 4096), "fp8_prefill_gate_up": (2048, 11008, 4096)}


class PreparedFp8:
    """8-bit float GEMM: A ~ normal(0, 1) and B ~ normal(0, 0.02) (seed 0)
    rounded to E4M3, per-tensor scales 1, rotated across copies."""

    def __init__(self, name: str, seed: int = 0):
        import torch
        from roofline_driven_optimisation_amd.inputs import f32_to_fp8_bits
        self.name = name
        self.M, self.N, self.K = FP8[name]
        rng = np.random.default_rng(seed)
        a = f32_to_fp8_bits(rng.standard_normal((self.M, self.K)).astype(np.float32), 0)
        b = f32_to_fp8_bits((rng.standard_normal((self.N, self.K)) * 0.02).astype(np.float32), 0)
        A, B = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
        C = torch.zeros(self.M, self.N, dtype=torch.float32, device="cuda")
        per_set = A.numel() + B.numel() + 4 * C.numel()
        self.sets = max(1, -(-ROTATE_BYTES // per_set))
        self.bufs = [(A, B, C)] + [(A.clone(), B.clone(), C.clone()) for _ in range(self.sets - 1)]
        self.rf = rl.gemm_roofline(self.M, self.N, self.K, "fp8", False)

    def launch(self, i: int, naive: bool = False):
        from roofline_driven_optimisation_amd import binding
        A, B, C = self.bufs[i % self.sets]
        binding.gemm_fp8(A, B, C, 1.0, 0.0, fmt=binding.FP8_E4M3)

    def rows_for(self, budget_flop):
        return sample_rows(self.M, self.N, self.K, budget_flop)

    def verify_launch(self, rows):
        import torch
        A, B, C = self.bufs[0]
        self.launch(0)
        torch.cuda.synchronize()
        self.a_host, self.b_host = A.cpu().numpy(), B.cpu().numpy()
        return C[torch.from_numpy(rows).cuda()].cpu().numpy()

    def oracle_rows(self, rows):
        import oracle
        ref, den = oracle.gemm_fp8(self.a_host[rows], self.b_host, None, 1.0, 0.0, 1.0, 1.0, 0)
        return ref, den, 2.0 * len(rows) * self.N * self.K

    def tolerance(self):
        # the matrix-core kernel's summation: each group of 8 consecutive
        # products loses under 7 * 2^-13 of its largest |product| (the
        # instruction drops bits 13 below it), then at most 8 ceil(K / 64)
        # + 3 fp32 roundings (the 8-bit products themselves are exact)
        return 7 * 2.0 ** -13 + (8 * -(-self.K // 64) + 3) * 2.0 ** -23

    def kernel_name(self) -> str:
        from roofline_driven_optimisation_amd import binding
        self.launch(0)
        return binding.last_kernel()


def prepare(name: str):
    if name in FP8:
        return PreparedFp8(name)
    if name.startswith("sum_"):
        return PreparedSum(name)
    if name in ATTENTION:
        return PreparedBatched(name)
    return Prepared(name)


SETTLE_S = 0.1  # minimum untimed warm-up, seconds
CLOCK_SAMPLE_S = 3.0  # the headline's clock and power loop, seconds


_MARKER = []


def phase_marker(closing: bool = False):
    """One launch of the library's smallest kernel, a K = 0 GEMM (C = 0 * C),
    outside any timed region: on a 1 x 8 C (one workgroup) just before a
    timed loop, on a 1 x 512 C (two workgroups) just after it.  In a kernel
    trace the pair encloses exactly a workload's timed launches, which
    would otherwise run together with its warm-up and what follows.  main()
    makes the first calls at start-up: a first call allocates and sets up,
    and such a pause between a warm-up and its timed loop lets the clock
    move."""
    import torch
    from roofline_driven_optimisation_amd import binding
    if not _MARKER:
        _MARKER.extend([torch.zeros(1, 0, dtype=torch.bfloat16, device="cuda"),
                        torch.zeros(0, 512, dtype=torch.bfloat16, device="cuda"),
                        torch.zeros(1, 512, dtype=torch.float32, device="cuda")])
    A, B, C = _MARKER
    n = 512 if closing else 8
    binding.gemm(A, B[:, :n], C[:, :n], 1.0, 0.0)


def time_workload(p: Prepared, steps: int, warmup: int, naive: bool = False):
    """(wall seconds per step, event seconds per launch) over `steps` launches.

    The untimed warm-up is `warmup` launches and at least SETTLE_S seconds of
    them: right after the operands are staged the GPU has not reached the
    clock it holds under sustained load (bf16 4096^3 measured 130 us per
    launch after 20 launches, 118-119 us after 200 or more, as in a 6 s
    steady-state loop)."""
    import torch
    i = 0
    t0 = time.perf_counter()
    while i < warmup or time.perf_counter() - t0 < SETTLE_S:
        p.launch(i, naive)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    phase_marker()  # outside the timed region: it ends the warm-up in a trace
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        p.launch(i, naive)
    end.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    phase_marker(closing=True)  # after the timed region: it ends the timed launches in a trace
    torch.cuda.synchronize()
    event = start.elapsed_time(end) * 1e-3 / steps
    return wall, event


def summary(p, sec: float, kname: str) -> dict:
    tflops = p.rf.flops / sec / 1e12
    gbs = p.rf.nbytes / sec / 1e9
    if isinstance(p, PreparedSum):
        return {"workload": p.name, "n": p.n, "dtype": "f32", "kernel": kname,
                "us": round(sec * 1e6, 2), "gbs": round(gbs, 1), "bound": p.rf.bound,
                "frac": round(p.rf.fraction(sec), 4)}
    if isinstance(p, PreparedFp8):
        return {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "dtype": "fp8_e4m3",
                "kernel": kname, "us": round(sec * 1e6, 2), "tflops": round(tflops, 2),
                "bound": p.rf.bound, "roofline_tflops": round(p.rf.attainable / 1e12, 1),
                "frac": round(p.rf.fraction(sec), 4)}
    if isinstance(p, PreparedBatched):
        return {"workload": p.name, "batch": p.batch, "M": p.M, "N": p.N, "K": p.K,
                "trans_b": p.trans_b, "dtype": "bf16", "kernel": kname,
                "us": round(sec * 1e6, 2), "tflops": round(tflops, 2), "gbs": round(gbs, 1),
                "bound": p.rf.bound, "roofline_tflops": round(p.rf.attainable / 1e12, 1),
                "frac": round(p.rf.fraction(sec), 4)}
    return {
        "workload": p.name, "M": p.w.M, "N": p.w.N, "K": p.w.K, "dtype": p.w.dtype,
        "alpha": p.w.alpha, "beta": p.w.beta, "kernel": kname, "us": round(sec * 1e6, 2),
        "tflops": round(tflops, 2), "gbs": round(gbs, 1), "bound": p.rf.bound,
        "roofline_tflops": round(p.rf.attainable / 1e12, 1),
        "frac": round(p.rf.fraction(sec), 4),
    }


def stream_probe(nbytes: int, copy: bool = False, steps: int = 100, warmup: int = 50,
                 grids=(512, 1024, 2048, 4096)) -> dict:
    """The library's device bandwidth probe (gemm_probe_stream) on `nbytes`:
    a flat streaming read (or copy) of that many bytes, rotated over enough
    buffers to exceed the last-level cache like the GEMM operands, event-timed
    for each grid size; the best is the practical floor for a kernel that
    reads the same bytes once."""
    import torch
    from roofline_driven_optimisation_amd import binding
    sets = max(1, -(-ROTATE_BYTES // nbytes))
    bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device="cuda")
            for i in range(sets)]
    dsts = [torch.empty_like(b) for b in bufs] if copy else None
    out = torch.empty(max(grids), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def run(i, g):
        binding.probe_stream(bufs[i % sets], out=out, dst=dsts[i % sets] if copy else None,
                             blocks=g, stream=stream)

    per = {}
    for g in grids:
        for i in range(warmup):
            run(i, g)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            run(i, g)
        end.record(stream)
        torch.cuda.synchronize()
        per[g] = start.elapsed_time(end) * 1e3 / steps
    best = min(per, key=per.get)
    moved = nbytes * (2 if copy else 1)
    del bufs, dsts
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "kind": "copy" if copy else "read", "us": round(per[best], 2),
            "tbs": round(moved / per[best] / 1e6, 3), "blocks": best,
            "us_by_blocks": {str(g): round(v, 2) for g, v in per.items()}}


def lds_bank_probe(strides=(1, 2, 4, 8, 16, 32, 64), steps: int = 4096, blocks: int = 512,
                   reps: int = 20) -> dict:
    """The library's shared-memory bank probe (gemm_probe_lds): time per
    launch, and per 4-byte read of one wave, for lane strides that put 1, 2,
    4, ... 64 lanes of a wave on one of the 64 banks."""
    import torch
    from roofline_driven_optimisation_amd import binding
    out = torch.empty(blocks, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for st in strides:
        for _ in range(3):
            binding.probe_lds(st, steps, out, blocks=blocks, stream=stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(reps):
            binding.probe_lds(st, steps, out, blocks=blocks, stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        us = start.elapsed_time(end) * 1e3 / reps
        res[str(st)] = {"us": round(us, 2),
                        "lanes_per_bank": math.gcd(st, 64)}
    base = res[str(strides[0])]["us"]
    for v in res.values():
        v["slowdown"] = round(v["us"] / base, 2)
    return {"steps": steps, "blocks": blocks, "by_stride": res}


def launch_floor(per_graph: int = 200, replays: int = 10) -> dict:
    """GPU-side cost of one launch: the library's smallest kernel (gemm_bf16
    with K = 0 on a 1 x 8 C, i.e. C = 0 * C, one workgroup) captured
    `per_graph` times into a graph, replayed and event-timed.  Host launch
    overhead is excluded (from Python a direct call takes several times
    longer than this), so it is what every launch costs the GPU itself, a
    floor under any event-timed kernel of a few microseconds; the decode
    entries report their HBM roofline fraction with and without it.  Each
    replay is checked (C must read zero)."""
    import torch
    from roofline_driven_optimisation_amd import binding
    A = torch.zeros(1, 0, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(0, 8, dtype=torch.bfloat16, device="cuda")
    C = torch.ones(1, 8, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.gemm(A, B, C, 1.0, 0.0)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(per_graph):
            binding.gemm(A, B, C, 1.0, 0.0)
    kname = binding.last_kernel()
    for _ in range(3):
        C.fill_(1.0)
        g.replay()
        torch.cuda.synchronize()
        if not bool(torch.all(C == 0.0)):
            raise RuntimeError("launch floor: graph replay gave a wrong C")
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / (replays * per_graph)
    return {"us": round(us, 2), "kernel": kname,
            "method": "graph of %d launches of C = 0*C (1x8, K = 0), %d replays, event-timed"
                      % (per_graph, replays)}


# Figures the pages quote, for context only (other machines; no MI355X number
# exists in them, so vs_baseline stays null).
PAGE_CONTEXT = {
    "rtx_a6000_fp32_4092": {"naive_row_major_gflops": 309, "naive_coalesced_gflops": 1986,
                            "cublas_gflops": 23250, "source": "Boehm SGEMM worklog, as quoted"},
    "h100_sxm5_spec": {"fp32_tflops": 67, "bf16_dense_tflops": 989, "hbm_tbs": 3.35},
}


def naive_ladder(steps: int = 3) -> dict:
    """The first rung of the optimisation ladder: one thread per output, no
    data reuse beyond the caches, on fp32 4092^3 (alpha 1.5, beta 0.5), next
    to the tiled kernel on the same workload."""
    p = Prepared("f32_4092")
    _, naive_s = time_workload(p, steps, 1, naive=True)
    _, tiled_s = time_workload(p, 20, 3)
    out = {"workload": "f32_4092", "naive_us": round(naive_s * 1e6, 1),
           "naive_tflops": round(p.rf.flops / naive_s / 1e12, 2),
           "tiled_us": round(tiled_s * 1e6, 1),
           "tiled_tflops": round(p.rf.flops / tiled_s / 1e12, 2),
           "speedup": round(naive_s / tiled_s, 1)}
    del p
    return out


def sample_smi():
    """One amd-smi reading of the GFX clock (XCD 0) and socket power, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--power"],
                           capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.TimeoutExpired):
        return None
    clk = re.search(r"GFX_0:\s*\n\s*CLK:\s*([0-9.]+)", r.stdout)
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)", r.stdout)
    if not clk or not pw:
        return None
    return {"gfx0_clock_mhz": float(clk.group(1)), "socket_power_w": float(pw.group(1))}


def sustain(name: str, seconds: float, p=None) -> dict:
    """Launch one workload back to back for `seconds` while amd-smi samples the
    clock and board power (steady state: power- and thermally-settled); `p`
    is the prepared workload, else it is prepared here."""
    import threading
    import torch
    if p is None:
        p = prepare(name)
    kname = p.kernel_name()
    samples = []

    def sampler():
        time.sleep(min(1.0, seconds / 4))
        while not done.is_set():
            s = sample_smi()
            if s:
                samples.append(s)
            done.wait(0.5)

    done = threading.Event()
    th = threading.Thread(target=sampler)
    th.start()
    n = 0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    while time.perf_counter() - t0 < seconds:
        for i in range(100):
            p.launch(n + i)
        n += 100
        torch.cuda.synchronize()
    end.record()
    torch.cuda.synchronize()
    done.set()
    th.join()
    sec = start.elapsed_time(end) * 1e-3 / n
    return {"workload": name, "kernel": kname, "launches": n, "us": round(sec * 1e6, 2),
            "tflops": round(p.rf.flops / sec / 1e12, 2), "smi_samples": samples}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# BASELINE configurations each GEMM workload belongs to (1: fp32 256^3; 2:
# fp32 4096^3 and 4092^3; 3: bf16 4096^3; 4: LLaMA-7B prefill; 5: decode)
CONFIG_OF = {"f32_256": 1, "f32_4096": 2, "f32_4092": 2, "bf16_4096": 3, "prefill_qkv": 4,
             "prefill_o": 4, "prefill_gate_up": 4, "prefill_down": 4, "decode_up_m1": 5,
             "decode_up_m8": 5, "decode_up_m16": 5, "decode_down_m1": 5, "decode_down_m8": 5,
             "decode_down_m16": 5, "decode_lm_head": 5}
CPU_SECONDS_PER_WORKLOAD = 1.2  # oracle time per sampled workload (the headline runs whole)


def verify(p, seconds) -> dict:
    """One launch outside the timed region keeps the GPU output's rows; the
    oracle, timed on four of them, sets how many rows fit in `seconds` of
    oracle time (all of them with an infinite budget); the operands on the
    GPU are then freed."""
    import torch
    every = p.rows_for(float("inf"))
    got = p.verify_launch(every)
    p.bufs = None
    if hasattr(p, "C0"):
        p.C0 = None
    torch.cuda.empty_cache()
    rows = every
    if every is not None and seconds != float("inf") and len(every) > 16:
        t0 = time.perf_counter()
        _, _, flop = p.oracle_rows(every[:4])
        rate = flop / max(time.perf_counter() - t0, 1e-6)
        rows = p.rows_for(seconds * rate)
        got = got[rows]
    return {"p": p, "rows": rows, "got": got}


def cpu_leg(records) -> tuple:
    """The CPU oracle, as it stands, on the sampled rows of every workload:
    its time is the CPU baseline (per BASELINE configuration; configuration
    1 also single-threaded) and its output is the reference for the parity
    of the GPU rows kept by verify().  Returns (cpu_baseline, {workload:
    parity})."""
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    per, parity = [], {}
    head = None
    for name, rec in records:
        p, rows = rec["p"], rec["rows"]
        t0 = time.perf_counter()
        ref, den, flop = p.oracle_rows(rows)
        t = time.perf_counter() - t0
        err = oracle.parity_error(rec["got"], ref, den)
        tol = p.tolerance()
        nrows = 1 if rows is None else len(rows)
        total_rows = 1 if rows is None else (p.w.M if hasattr(p, "w") else p.M)
        parity[name] = {"outputs_checked": int(np.size(rec["got"])),
                        "rows": ("all %d" % total_rows if nrows == total_rows else
                                 "%d of %d (leading and trailing)" % (nrows, total_rows))
                        if rows is not None else "the sum",
                        "err": float("%.3e" % err), "tol": float("%.3e" % tol),
                        "ok": bool(err <= tol)}
        entry = {"workload": name, "config": CONFIG_OF.get(name), "rows": nrows,
                 "of_rows": total_rows, "seconds": round(t, 3),
                 "gflops": round(flop / t / 1e9, 2), "threads": threads}
        per.append(entry)
        if name == HEADLINE:
            head = entry
        if name == "f32_256":
            oracle.set_num_threads(1)
            t0 = time.perf_counter()
            p.oracle_rows(rows)
            t1 = time.perf_counter() - t0
            oracle.set_num_threads(threads)
            entry["single_thread"] = {"seconds": round(t1, 4),
                                      "gflops": round(flop / t1 / 1e9, 3), "threads": 1}
    out = {"value": round(2.0 * head["rows"] * 4096 * 4096 / head["seconds"] / 1e12, 6),
           "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": "rows 0..%d of the bf16 4096^3 GEMM (all %d x 4096 outputs, K=4096), "
                     "fp64 i-k-j loop, %.1f s; per_config: the oracle on sampled rows of every "
                     "workload (%.1f s each at most)" % (head["rows"] - 1, head["rows"],
                                                        head["seconds"],
                                                        CPU_SECONDS_PER_WORKLOAD),
           "per_config": per, "cpu": cpu_model(), "logical_cpus": os.cpu_count()}
    return out, parity


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--secondary-steps", type=int, default=50)
    ap.add_argument("--only", default="", help="comma-separated workloads to time "
                    "(profiling runs); skips the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ladder", action="store_true",
                    help="skip the naive-kernel rung (fp32 4092^3)")
    ap.add_argument("--sustain", type=float, default=0.0, metavar="SECONDS",
                    help="only launch the --only workloads (default: the headline) back to "
                    "back for SECONDS each, sampling clock and power with amd-smi")
    ap.add_argument("--probes", action="store_true",
                    help="only run the library's bandwidth and LDS bank probes (one JSON line "
                    "each; for profiling them)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, --steps times "
                    "(calibrates the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs on a single MI355X and has "
              "no multi-GPU path (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    # the phase marker's tensors and the library's first K = 0 call, made
    # here so that no first-use pause falls between a warm-up and its timed
    # launches
    phase_marker()
    phase_marker(closing=True)
    torch.cuda.synchronize()

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.warmup)):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / args.steps
        log(json.dumps({"copy_mib": args.copy_probe, "us": round(sec * 1e6, 2),
                        "gbs_read_plus_write": round(2 * n / sec / 1e9, 1)}))
        return

    if args.probes:
        log(json.dumps({"read_4096x11008_bf16": stream_probe(4096 * 11008 * 2, steps=args.steps,
                                                             warmup=args.warmup)}))
        log(json.dumps({"lds_bank_probe": lds_bank_probe(reps=args.steps)}))
        return

    if args.sustain > 0:
        for name in (args.only or HEADLINE).split(","):
            log(json.dumps(sustain(name, args.sustain)))
        return

    if args.only:
        for name in args.only.split(","):
            p = prepare(name)
            kname = p.kernel_name()
            wall, ev = time_workload(p, args.steps, args.warmup)
            log(json.dumps(summary(p, ev, kname)))
        return

    cpu = not args.no_cpu_baseline
    log("bench: preparing %s" % HEADLINE)
    head = Prepared(HEADLINE)
    kname = head.kernel_name()
    log("bench: timing %s (%s), %d steps" % (HEADLINE, kname, args.steps))
    wall, ev = time_workload(head, args.steps, args.warmup)
    # the clock and power the headline holds, from a short back-to-back loop
    # after (not inside) the timed steps
    held = sustain(HEADLINE, CLOCK_SAMPLE_S, head)
    smi = held["smi_samples"]
    clock = {"how": "amd-smi, every 0.5 s of a %.1f s back-to-back loop of the headline "
                    "after its timed steps" % CLOCK_SAMPLE_S, "us_in_loop": held["us"]}
    if smi:
        # median over the samples, and their range (a sample can fall on a
        # moment between the loop's batches)
        for key, out in (("gfx0_clock_mhz", "gfx_clock_mhz"), ("socket_power_w", "socket_power_w")):
            vals = sorted(x[key] for x in smi)
            clock[out] = vals[len(vals) // 2]
            clock[out + "_range"] = [vals[0], vals[-1]]
    log("bench: clock " + json.dumps(clock))
    records = []
    head_rf = head.rf
    if cpu:
        records.append((HEADLINE, verify(head, float("inf"))))

    also = []
    for name in SECONDARY:
        log("bench: secondary %s" % name)
        p = prepare(name)
        kn = p.kernel_name()
        _, sec = time_workload(p, args.secondary_steps, max(3, args.warmup // 4))
        s = summary(p, sec, kn)
        if isinstance(p, PreparedSum):
            # the page's first version beside it (the ladder's other rung)
            _, nsec = time_workload(p, max(3, args.secondary_steps // 4), 3, naive=True)
            s["naive_us"] = round(nsec * 1e6, 2)
            s["naive_gbs"] = round(p.rf.nbytes / nsec / 1e9, 1)
        log("  " + json.dumps(s))
        also.append(s)
        if cpu:
            records.append((name, verify(p, CPU_SECONDS_PER_WORKLOAD)))
        del p
        torch.cuda.empty_cache()
    if cpu:  # configuration 1 (fp32 256^3) is a parity configuration, not timed
        records.append(("f32_256", verify(prepare("f32_256"), float("inf"))))

    # fused-epilogue entries: the plain GEMM of the same shape beside them
    plain = {s_["workload"]: s_["us"] for s_ in also}
    for s_ in also:
        base = s_["workload"].partition("+")[0]
        if base != s_["workload"] and base in plain:
            s_["plain_us"] = plain[base]
            s_["epilogue_us"] = round(s_["us"] - plain[base], 2)

    floor = launch_floor()
    log("bench: launch floor " + json.dumps(floor))
    # the flat-read floor of the decode GEMMs' weight bytes, and a copy
    probes = {"read_4096x11008_bf16": stream_probe(4096 * 11008 * 2),
              "read_4096x32000_bf16": stream_probe(4096 * 32000 * 2),
              "copy_1GiB": stream_probe(1 << 30, copy=True)}
    log("bench: bandwidth probes " + json.dumps(probes))
    lds = lds_bank_probe()
    log("bench: shared-memory bank probe " + json.dumps(lds))
    flat = {v["bytes"]: v["us"] for k, v in probes.items() if v["kind"] == "read"}
    for s_ in also:
        if s_["bound"] == "hbm" and "K" in s_ and s_["K"] * s_["N"] * 2 in flat:
            # the same weight bytes read flat: the floor this kernel is held to
            s_["flat_read_us"] = flat[s_["K"] * s_["N"] * 2]
            s_["vs_flat_read"] = round(s_["flat_read_us"] / s_["us"], 4)
    for s_ in also:
        if s_["bound"] == "hbm":
            body = s_["us"] - floor["us"]
            s_["frac_excl_launch_floor"] = round(s_["frac"] * s_["us"] / body, 4) if body > 0 else None

    ladder = None
    if not args.no_ladder:
        log("bench: naive rung, fp32 4092^3")
        ladder = naive_ladder()
        log("  " + json.dumps(ladder))

    traffic = stored_traffic(kname, HEADLINE)
    achieved = head_rf.flops / ev / 1e12
    peak = rl.MI355X_PEAK_BF16 / 1e12
    result = {
        "metric": "GEMM TFLOP/s and % of roofline at M=N=K=4096 (fp32, bf16) + skinny-M GB/s",
        "value": round(head_rf.flops / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: A, B ~ normal(0, 1/64) rounded to bf16, seed 0",
        "config": {"workload": "bf16-input fp32-accumulate GEMM M=N=K=4096, alpha=1, beta=0, "
                               "row-major, C fp32", "kernel": kname,
                   "rotated_operand_sets": head.sets, "warmup_min_s": SETTLE_S},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic},
        "also": also,
        "clock": clock,
        "launch_floor": floor,
        "bandwidth_probes": probes,
        "lds_bank_probe": lds,
        "ladder": ladder,
        "page_context": PAGE_CONTEXT,
    }
    if cpu:
        log("bench: CPU oracle on the sampled rows (baseline and parity)")
        result["cpu_baseline"], parity = cpu_leg(records)
        result["parity"] = parity.pop(HEADLINE)
        for s_ in also:
            s_["parity"] = parity.get(s_["workload"])
        result["parity_f32_256"] = parity.get("f32_256")
        log("bench: parity " + json.dumps({k: v["ok"] for k, v in parity.items()}))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
