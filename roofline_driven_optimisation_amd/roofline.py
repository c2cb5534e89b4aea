"""Roofline arithmetic: FLOPs, bytes, arithmetic intensity, ridge and bound.

The model is the one the pages build up:

* a multiply-add counts as 2 FLOPs, so a GEMM does 2*M*N*K FLOPs
  (page "Naive GEMM and Roofline analysis", sections 10.1 and 10.3.1);
* arithmetic intensity AI = FLOPs / bytes moved (page "From model computation
  to GPU execution", section 5.1);
* the attainable performance is min(P_compute, BW * AI) and the ridge point
  is P_compute / BW (same page, section 5.2; page "Memory hierarchy and cost
  table", section 4.6; page "Where kernel performance comes from", roofline
  section);
* the HBM-level bytes of a GEMM with perfect on-chip reuse are A and B read
  once and C written once, plus C read once more when beta != 0 (section
  10.3.1, and the GEMM subsection of "Where kernel performance comes from",
  which drops the C read when beta = 0).

MI355X peaks are AMD's published figures, not the pages': dense bf16 MFMA
2516.6 TFLOP/s (256 CUs x 2.4 GHz x 4096 FLOP per CU per clock), fp8 twice
that (5033 TFLOP/s), fp32
157.3 TFLOP/s, HBM3E 8.0 TB/s.
"""
from __future__ import annotations

from dataclasses import dataclass

# ---- MI355X (gfx950) published peaks -------------------------------------
MI355X_CUS = 256
MI355X_CLOCK_HZ = 2.4e9
MI355X_BF16_FLOP_PER_CLK_PER_CU = 4096
MI355X_PEAK_BF16 = MI355X_CUS * MI355X_CLOCK_HZ * MI355X_BF16_FLOP_PER_CLK_PER_CU  # 2.5166e15
MI355X_PEAK_FP8 = 2 * MI355X_PEAK_BF16  # 8-bit float MFMA: twice the bf16 rate
MI355X_PEAK_FP32 = 157.3e12
MI355X_PEAK_HBM = 8.0e12  # bytes/s

ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1}


def gemm_flops(M: int, N: int, K: int) -> int:
    """2*M*N*K: one multiply and one add per (m, n, k)."""
    return 2 * M * N * K


def gemm_bytes(M: int, N: int, K: int, in_bytes: int, out_bytes: int = 4,
               beta_nonzero: bool = False) -> int:
    """Compulsory HBM bytes: A and B read once, C written once (and read once
    more when beta != 0)."""
    return in_bytes * (M * K + K * N) + out_bytes * M * N * (2 if beta_nonzero else 1)


def arithmetic_intensity(flops: float, nbytes: float) -> float:
    return flops / nbytes


def gemm_ai(M: int, N: int, K: int, in_bytes: int, out_bytes: int = 4,
            beta_nonzero: bool = False) -> float:
    return gemm_flops(M, N, K) / gemm_bytes(M, N, K, in_bytes, out_bytes, beta_nonzero)


def naive_thread_ai(K: int, elem_bytes: int = 4) -> float:
    """Per-thread AI of the one-thread-per-output kernel: 2K FLOPs against a
    row of A, a column of B and one C write, 2K / (8K + 4) for fp32."""
    return (2.0 * K) / (elem_bytes * (2 * K + 1))


def per_instruction_ai(tm: int, tn: int, elem_bytes: int = 4) -> float:
    """AI counted per load instruction for a TM x TN register tile: each k
    step loads TM + TN elements and does TM*TN multiply-adds."""
    return (2.0 * tm * tn) / (elem_bytes * (tm + tn))


def reuse_factor(tile_m: int, tile_n: int) -> float:
    """Multiply-adds per element loaded per k column for a tile_m x tile_n
    output tile (the reuse ratios of section 10.4.1)."""
    return (tile_m * tile_n) / float(tile_m + tile_n)


def cta_stage_ai(bm: int, bn: int, bk: int, elem_bytes: int) -> float:
    """A/B global-memory AI of one K stage of a BM x BN tile (C ignored):
    2*BM*BN*BK FLOPs over elem_bytes*(BM*BK + BK*BN) bytes."""
    return (2.0 * bm * bn * bk) / (elem_bytes * (bm * bk + bk * bn))


def ridge(peak_flops: float, bandwidth: float) -> float:
    return peak_flops / bandwidth


def attainable(peak_flops: float, bandwidth: float, ai: float) -> float:
    """min(P_compute, BW * AI)."""
    return min(peak_flops, bandwidth * ai)


def mma_flops(m: int, n: int, k: int) -> int:
    return 2 * m * n * k


def tensor_peak(units: int, clock_hz: float, flop_per_clk_per_unit: float) -> float:
    return units * clock_hz * flop_per_clk_per_unit


def llama7b_decode_flops(context: int, d: int = 4096, layers: int = 32,
                         ffn: int = 11008, vocab: int = 32000):
    """FLOPs of one decoded token of a LLaMA-7B-shaped model.

    Returns (weight_gemm_flops, attention_flops): the weight GEMMs are QKV
    (d x 3d), O (d x d), FFN gate/up/down (3 x d x ffn) per layer plus the
    LM head (d x vocab); attention is QK^T and PV against ``context`` keys,
    2*d*context multiply-adds per layer.
    """
    per_layer = 3 * d * d + d * d + 3 * d * ffn
    weights = 2 * (layers * per_layer + d * vocab)
    attention = 2 * layers * 2 * d * context
    return weights, attention


@dataclass
class Roofline:
    """Where one GEMM sits on the MI355X roofline."""

    flops: int
    nbytes: int
    ai: float
    peak_compute: float
    peak_bw: float
    bound: str  # "mfma" (bf16 or fp8 matrix cores), "fp32" (fp32 compute) or "hbm"
    attainable: float

    def fraction(self, seconds: float) -> float:
        return (self.flops / seconds) / self.attainable

    def hbm_fraction(self, seconds: float) -> float:
        return (self.nbytes / seconds) / self.peak_bw


def gemm_roofline(M: int, N: int, K: int, dtype: str, beta_nonzero: bool,
                  bias: bool = False) -> Roofline:
    """Roofline position of a GEMM with fp32 output on MI355X.  With ``bias``
    (the fused Linear-layer epilogue) the N fp32 bias values join the bytes;
    the epilogue's per-element add and activation are not counted as FLOPs
    (M N of them against 2 M N K)."""
    in_bytes = ELEM_BYTES[dtype]
    flops = gemm_flops(M, N, K)
    nbytes = gemm_bytes(M, N, K, in_bytes, 4, beta_nonzero) + (4 * N if bias else 0)
    peak = {"bf16": MI355X_PEAK_BF16, "fp8": MI355X_PEAK_FP8}.get(dtype, MI355X_PEAK_FP32)
    ai = flops / nbytes
    att = attainable(peak, MI355X_PEAK_HBM, ai)
    if MI355X_PEAK_HBM * ai < peak:
        bound = "hbm"
    else:
        bound = "mfma" if dtype in ("bf16", "fp8") else "fp32"
    return Roofline(flops, nbytes, ai, peak, MI355X_PEAK_HBM, bound, att)


def sum_roofline(n: int) -> Roofline:
    """Roofline position of summing n float32 values (page "Memory hierarchy
    and cost table", section 4.7): n - 1 additions (counted as n) against 4n
    bytes read and one float written, AI 1/4, far left of every ridge, so
    HBM-bound.  The fp32 VALU peak is the compute roof."""
    flops = max(n, 1)
    nbytes = 4 * n + 4
    ai = flops / nbytes
    return Roofline(flops, nbytes, ai, MI355X_PEAK_FP32, MI355X_PEAK_HBM, "hbm",
                    attainable(MI355X_PEAK_FP32, MI355X_PEAK_HBM, ai))


def batched_gemm_roofline(batch: int, M: int, N: int, K: int, dtype: str) -> Roofline:
    """A batch of independent GEMMs (beta = 0, fp32 C): batch times the
    FLOPs and compulsory bytes of one.  Attention's S = Q K^T with d = 128
    lands left of the ridge: writing the fp32 scores outweighs the MFMA work."""
    one = gemm_roofline(M, N, K, dtype, False)
    flops = batch * one.flops
    nbytes = batch * one.nbytes
    ai = flops / nbytes
    peak = one.peak_compute
    att = attainable(peak, MI355X_PEAK_HBM, ai)
    bound = "hbm" if MI355X_PEAK_HBM * ai < peak else one.bound
    return Roofline(flops, nbytes, ai, peak, MI355X_PEAK_HBM, bound, att)
