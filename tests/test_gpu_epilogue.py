"""GPU parity of the fused Linear-layer epilogue, C = act(alpha*A*B + beta*C +
bias[n]), through the C ABI (gemm_bf16_bias_act / gemm_f32_bias_act),
against the CPU oracle's epilogue, on every kernel family the dispatcher can
pick: the four-wave and ping-pong 256 x 256 kernels (whole tiles and the
split last round), the smaller bf16 tiles, the decode kernel (one split,
XCD-local and uncached reductions), the fp32 kernels, the naive fallback and
the K = 0 path.  Random inputs are held to the parity tolerance on the
epilogue's denominator; integer inputs with identity or ReLU are exact."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, log, sample_positions, to_device
from roofline_driven_optimisation_amd import binding
from roofline_driven_optimisation_amd.inputs import make_bias, make_case

pytestmark = pytest.mark.gpu

ACTS = [binding.ACT_NONE, binding.ACT_RELU, binding.ACT_GELU, binding.ACT_SILU]
ACT_IDS = ["none", "relu", "gelu", "silu"]


def run_epi(case, bias, act, env=None, monkeypatch=None):
    import torch
    for k, v in (env or {}).items():
        monkeypatch.setenv(k, v)
    A, B, C = to_device(case)
    b = torch.from_numpy(bias).cuda() if bias is not None else None
    log("  gpu epilogue %s %dx%dx%d %s alpha=%g beta=%g act=%d bias=%s env=%s" % (
        case.name, case.M, case.N, case.K, case.dtype, case.alpha, case.beta, act,
        bias is not None, env))
    fn = binding.gemm_bf16_bias_act if case.bf16 else binding.gemm_f32_bias_act
    fn(A, B, C, b, act, case.alpha, case.beta)
    name = binding.last_kernel()
    torch.cuda.synchronize()
    return C.cpu().numpy(), name


def check(case, got, bias, act, sampled=False):
    if sampled:
        rows, cols = sample_positions(case.M, case.N, 1024, seed=3)
        ref, den = oracle.gemm_entries(case.A, case.B, rows, cols, case.C, case.alpha,
                                       case.beta, bf16=case.bf16, bias=bias, act=act)
        err = oracle.parity_error(got[rows, cols], ref, den)
    else:
        ref, den = oracle.gemm(case.A, case.B, case.C, case.alpha, case.beta, bf16=case.bf16,
                               bias=bias, act=act)
        err = oracle.parity_error(got, ref, den)
    log("  epilogue parity %s act=%d err=%.3e" % (case.name, act, err))
    assert err <= TOL[case.dtype], (case.name, act, err)


# (shape, env, expected kernel-name prefix): one entry per kernel path
BF16_PATHS = [
    ((512, 768, 320), {"MGEMM_BF16_TILE": "bf16_q4_256x256x32", "MGEMM_PP_SPLIT": "0"},
     "bf16_q4_256x256x32"),
    ((520, 776, 328), {"MGEMM_BF16_TILE": "bf16_q4_256x256x32"}, "bf16_q4_256x256x32_splitk"),
    ((1024, 4096, 264), {"MGEMM_BF16_TILE": "bf16_q4_256x256x32"},
     "bf16_q4_256x256x32_splitk_xcd"),
    ((520, 776, 328), {"MGEMM_BF16_TILE": "bf16_pp_256x256x32"}, "bf16_pp_256x256x32_splitk"),
    ((512, 768, 320), {"MGEMM_BF16_TILE": "bf16_pp_256x256x32", "MGEMM_PP_SPLIT": "0"},
     "bf16_pp_256x256x32"),
    ((512, 768, 320), {"MGEMM_BF16_TILE": "bf16_q16_256x256x32", "MGEMM_PP_SPLIT": "0"},
     "bf16_q16_256x256x32"),
    ((520, 776, 328), {"MGEMM_BF16_TILE": "bf16_q16_256x256x32"}, "bf16_q16_256x256x32_splitk"),
    ((1024, 4096, 264), {"MGEMM_BF16_TILE": "bf16_q16_256x256x32"},
     "bf16_q16_256x256x32_splitk_xcd"),
    ((300, 264, 200), {"MGEMM_BF16_TILE": "bf16_mfma_256x128x64"}, "bf16_mfma_256x128x64"),
    ((300, 264, 200), {"MGEMM_BF16_TILE": "bf16_mfma_128x256x64"}, "bf16_mfma_128x256x64"),
    ((300, 264, 200), {"MGEMM_BF16_TILE": "bf16_mfma_128x128x64"}, "bf16_mfma_128x128x64"),
    ((1, 4096, 1024), {}, "skinny_bf16"),
    ((16, 4096, 4096), {}, "skinny_bf16_splitk_xcd"),
    ((16, 896, 4096), {}, "skinny_bf16_splitk"),
    ((5, 1160, 2048), {"MGEMM_SKINNY_SPLITS": "1"}, "skinny_bf16"),
    ((37, 100, 60), {}, "naive_bf16"),
    ((40, 72, 0), {}, "scale_c"),
]


@pytest.mark.parametrize("act", ACTS, ids=ACT_IDS)
@pytest.mark.parametrize("path", BF16_PATHS, ids=lambda p: p[2] + "_" + "x".join(map(str, p[0])))
def test_bf16_epilogue(path, act, monkeypatch):
    (M, N, K), env, want = path
    beta = 0.5 if act in (binding.ACT_RELU, binding.ACT_SILU) else 0.0
    case = make_case(M, N, K, "bf16", 1.25, beta, "n:1", "n:0.05", "n:1", seed=70 + act)
    bias = make_bias(N, "n:0.5", seed=71)
    got, name = run_epi(case, bias, act, env, monkeypatch)
    assert name.startswith(want), (name, want)
    if want.startswith("bf16_mfma") or want.startswith("naive") or M * N <= 1 << 20:
        check(case, got, bias, act)
    else:
        check(case, got, bias, act, sampled=True)


F32_PATHS = [
    ((300, 264, 200), "f32_mfma_128x128x32_vec4"),   # direct-copy kernel (aligned rows)
    ((130, 250, 70), "f32_mfma_128x128x32_scalar"),  # staged kernel, N % 4 != 0
    ((33, 48, 0), "scale_c"),
]


@pytest.mark.parametrize("act", ACTS, ids=ACT_IDS)
@pytest.mark.parametrize("path", F32_PATHS, ids=lambda p: p[1] + "_" + "x".join(map(str, p[0])))
def test_f32_epilogue(path, act, monkeypatch):
    (M, N, K), want = path
    case = make_case(M, N, K, "f32", 1.5, 0.5, "u", "u", "u", seed=80 + act)
    bias = make_bias(N, "u", seed=81)
    got, name = run_epi(case, bias, act, None, monkeypatch)
    assert name == want, name
    check(case, got, bias, act)


@pytest.mark.parametrize("act", [binding.ACT_NONE, binding.ACT_RELU], ids=["none", "relu"])
@pytest.mark.parametrize("path", BF16_PATHS[:-2], ids=lambda p: p[2] + "_" + "x".join(map(str, p[0])))
def test_bf16_epilogue_exact_integers(path, act, monkeypatch):
    """Integer A, B, C and bias: every sum is exact in fp32, so identity and
    ReLU results equal the oracle's bit for bit."""
    (M, N, K), env, want = path
    case = make_case(M, N, K, "bf16", 1.0, 0.5, "i:4", "i:4", "i:4", seed=90)
    bias = make_bias(N, "i:8", seed=91)
    got, name = run_epi(case, bias, act, env, monkeypatch)
    assert name.startswith(want), name
    ref, _ = oracle.gemm(case.A, case.B, case.C, 1.0, 0.5, bf16=True, bias=bias, act=act)
    assert np.array_equal(got.astype(np.float64), ref)


def test_no_bias_matches_plain_gemm(monkeypatch):
    """bias NULL with no activation is the plain GEMM: identical bits."""
    import torch
    case = make_case(512, 768, 320, "bf16", 1.0, 0.0, "n:1", "n:0.05", seed=95)
    A, B, C1 = to_device(case)
    C2 = C1.clone()
    binding.gemm_bf16(A, B, C1)
    binding.gemm_bf16_bias_act(A, B, C2, None, binding.ACT_NONE)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def test_bias_only_and_activation_only(monkeypatch):
    """Each half of the epilogue alone: bias without activation, activation
    without bias."""
    case = make_case(300, 264, 200, "bf16", 1.0, 0.0, "n:1", "n:0.05", seed=96)
    bias = make_bias(264, "n:0.5", seed=97)
    got, _ = run_epi(case, bias, binding.ACT_NONE)
    check(case, got, bias, binding.ACT_NONE)
    got, _ = run_epi(case, None, binding.ACT_GELU)
    check(case, got, None, binding.ACT_GELU)


@pytest.mark.parametrize("name,act", [("prefill_gate_up", binding.ACT_GELU),
                                      ("decode_up_m1", binding.ACT_SILU)],
                         ids=["prefill_gate_up+bias_gelu", "decode_up_m1+bias_silu"])
def test_benchmarked_fused_workloads_full(name, act):
    """The two fused workloads the benchmark times, at full size with its
    inputs (the workload's operands, a normal(0, 0.5) bias, seed 0), every
    element against the oracle's epilogue."""
    from roofline_driven_optimisation_amd.inputs import workload
    w = workload(name)
    case = w.case(0)
    bias = make_bias(w.N, "n:0.5", 0)
    got, kname = run_epi(case, bias, act)
    log("  kernel %s" % kname)
    check(case, got, bias, act)


def test_bad_activation_rejected():
    import torch
    case = make_case(8, 8, 8, "bf16", seed=1)
    A, B, C = to_device(case, c_fill=0.0)
    with pytest.raises(binding.GemmError) as e:
        binding.gemm_bf16_bias_act(A, B, C, None, 4)
    assert e.value.status == 1
    assert binding.last_kernel() == "none"
    torch.cuda.synchronize()
