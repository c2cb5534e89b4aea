"""Pins for the roofline calculator against numbers the pages print (no GPU)."""
import math

import pytest

from roofline_driven_optimisation_amd import roofline as rl
from roofline_driven_optimisation_amd.inputs import WORKLOADS, workload


@pytest.fixture(scope="module")
def page(golden):
    rows = golden("page_numbers.txt")[None]
    return {k: float(v) for k, v in rows}


def test_naive_thread_ai(page):
    # 2K / (8K + 4) at K = 4096 -> 0.24997, "about 1/4"
    v = rl.naive_thread_ai(4096)
    assert abs(v - 2 * 4096 / (8 * 4096 + 4)) < 1e-15
    assert abs(v - page["naive_thread_ai_k4096"]) < 1e-3


def test_kernel_ai_fp32_4096(page):
    ai = rl.gemm_ai(4096, 4096, 4096, 4, 4, beta_nonzero=False)
    assert round(ai) == page["kernel_ai_fp32_4096"]
    assert abs(ai - 2 * 4096 / 12) < 1e-9


def test_ridges(page):
    assert round(rl.ridge(67e12, 3.35e12)) == page["ridge_h100_fp32"]
    assert round(rl.ridge(989e12, 3.35e12)) == page["ridge_h100_fp16"]
    assert rl.ridge(20e12, 500e9) == page["hyp_ridge"]
    assert rl.ridge(2e15, 8e12) == page["b200_ridge"]


def test_hypothetical_gpu_attainable(page):
    assert rl.attainable(20e12, 500e9, 10) / 1e12 == page["hyp_attainable_ai10_tflops"]
    assert rl.attainable(20e12, 500e9, 1) / 1e12 == page["hyp_attainable_ai1_tflops"]
    # right of the ridge the compute roof binds
    assert rl.attainable(20e12, 500e9, 100) == 20e12


def test_cta_stage_ai(page):
    assert 2 * 16 * 16 * 64 == page["tile_flops_16x16_bk64"]
    assert 2 * (16 * 64 + 64 * 16) == page["tile_bytes_16x16_bk64"]
    assert 2 * 64 * 64 * 64 == page["tile_flops_64x64_bk64"]
    assert 2 * (64 * 64 + 64 * 64) == page["tile_bytes_64x64_bk64"]
    assert rl.cta_stage_ai(16, 16, 64, 2) == page["tile_ai_16x16_bk64_bf16"]
    assert rl.cta_stage_ai(64, 64, 64, 2) == page["tile_ai_64x64_bk64_bf16"]
    # square tile: AI = B / s
    for b in (16, 64, 128, 256):
        assert rl.cta_stage_ai(b, b, 64, 2) == b / 2


def test_reuse_factors(page):
    assert rl.reuse_factor(128, 128) == page["reuse_block_128x128"]
    assert int(rl.reuse_factor(64, 32)) == page["reuse_warp_64x32"]
    # 8x8 register tile: 64 multiply-adds over 16 loads, each element used 8 times
    assert rl.reuse_factor(8, 8) * 2 == 8


def test_per_instruction_ai(page):
    assert rl.per_instruction_ai(1, 1) == page["per_instr_ai_naive"]
    assert rl.per_instruction_ai(4, 4) == page["per_instr_ai_tile4x4"]


def test_tensor_core_peak(page):
    assert rl.mma_flops(16, 8, 16) == page["mma_m16n8k16_flops"]
    assert round(rl.tensor_peak(132, 1.83e9, 4096) / 1e12) == page["h100_tc_peak_tflops"]


def test_square_fp16_ai(page):
    # beta = 0, 2-byte operands, output also 2 bytes: N/3 = 1365, "~1300"
    ai = rl.gemm_ai(4096, 4096, 4096, 2, 2, beta_nonzero=False)
    assert abs(ai - 4096 / 3) < 1e-9
    assert abs(ai - page["square_fp16_ai_4096"]) / page["square_fp16_ai_4096"] < 0.06


def test_llama7b_flops(page):
    w, a = rl.llama7b_decode_flops(2048)
    assert round(w / 1e9, 1) == page["llama7b_weight_gflops"]
    assert round(a / (w + a), 3) == page["llama7b_attn_share_2048"]
    w5, a5 = rl.llama7b_decode_flops(512)
    assert round(a5 / (w5 + a5), 2) == page["llama7b_attn_share_512"]
    w4, a4 = rl.llama7b_decode_flops(4096)
    assert round(a4 / (w4 + a4), 2) == page["llama7b_attn_share_4096"]


def test_tiling_read_counts(page):
    """Naive vs tiled logical reads, n x n product: n^2 outputs each read
    2n inputs, against 2 n^2 inputs read once."""
    for n, key in ((2, "2x2"), (4, "4x4")):
        assert n * n * 2 * n == page["tiling_reads_%s_naive" % key]
        assert 2 * n * n == page["tiling_reads_%s_tiled" % key]


def test_mi355x_peaks():
    assert abs(rl.MI355X_PEAK_BF16 - 2516.5824e12) < 1e6
    assert rl.ridge(rl.MI355X_PEAK_BF16, rl.MI355X_PEAK_HBM) == pytest.approx(314.57, rel=1e-4)
    assert rl.ridge(rl.MI355X_PEAK_FP32, rl.MI355X_PEAK_HBM) == pytest.approx(19.66, rel=1e-3)


def test_workload_rooflines():
    r = rl.gemm_roofline(4096, 4096, 4096, "bf16", False)
    assert r.bound == "mfma" and r.ai == pytest.approx(1024.0)
    assert r.flops / r.attainable == pytest.approx(54.6e-6, rel=1e-3)
    r = rl.gemm_roofline(4096, 4096, 4096, "f32", True)
    assert r.bound == "fp32" and r.ai == pytest.approx(512.0)
    for name in ("decode_up_m1", "decode_down_m16", "decode_lm_head"):
        w = workload(name)
        r = rl.gemm_roofline(w.M, w.N, w.K, w.dtype, w.beta != 0)
        assert r.bound == "hbm"
    w = workload("decode_lm_head")
    r = rl.gemm_roofline(w.M, w.N, w.K, w.dtype, False)
    assert r.nbytes == 2 * (4096 + 4096 * 32000) + 4 * 32000
    assert r.nbytes / r.peak_bw == pytest.approx(32.8e-6, rel=1e-2)


def test_workload_table():
    names = {w.name for w in WORKLOADS}
    assert {"f32_256", "f32_4096", "f32_4092", "bf16_4096", "prefill_qkv", "prefill_o",
            "prefill_gate_up", "prefill_down", "decode_lm_head"} <= names
    assert sum(1 for w in WORKLOADS if w.group == "decode") == 7
    assert workload("f32_4096").alpha == 1.5 and workload("f32_4096").beta == 0.5
    assert math.isclose(float(workload("bf16_4096").dist_a[2:]), 1 / 64)
