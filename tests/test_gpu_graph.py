"""The library under HIP graph capture (torch.cuda.graph), for the plain,
decode-shaped, 8-bit float and batched GEMMs.

Under capture the library allocates nothing, runs no placement probe and
never uses the ping-pong kernel's split tail (its flag epochs would be stale
on replays).  A decode-shaped call uses split-K scratch only when the
capturing stream already has it (the kernel leaves its counters re-armed, so
every replay starts clean); otherwise it runs with one split.  Each graph is
replayed several times with eager library work and synchronisations between
the replays, and every replay is checked exactly against the oracle
(integer inputs)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import to_device
from roofline_driven_optimisation_amd import binding
from roofline_driven_optimisation_amd.inputs import make_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.library()
    oracle.build(force=False)
    return torch


def capture_and_check(torch, case, stream, warm, want_prefix, replays=4):
    A, B, C = to_device(case)
    C0 = C.clone()
    ref, _ = oracle.gemm(case.A, case.B, case.C, case.alpha, case.beta, bf16=True)
    if warm:  # a direct call on the capturing stream first: its scratch exists
        with torch.cuda.stream(stream):
            binding.gemm(A, B, C, case.alpha, case.beta)
        stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        binding.gemm(A, B, C, case.alpha, case.beta)
    name = binding.last_kernel()
    assert name.startswith(want_prefix), name
    # eager work between replays, on another shape through the same library
    other = make_case(16, 1024, 512, "bf16", 1.0, 0.0, "i:4", "i:4", seed=81)
    oA, oB, oC = to_device(other)
    for r in range(replays):
        C.copy_(C0)
        g.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), (case.name, r)
        binding.gemm(oA, oB, oC, 1.0, 0.0)
        torch.cuda.synchronize()
    return name


@pytest.mark.parametrize("shape", [(16, 4096, 2048), (3, 1160, 2048), (1, 520, 4096)],
                         ids=lambda s: "x".join(map(str, s)))
def test_decode_split_scratch_existing(torch, shape):
    """Scratch allocated by a direct call on the stream before capture."""
    case = make_case(*shape, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=80)
    s = torch.cuda.Stream()
    name = capture_and_check(torch, case, s, warm=True, want_prefix="skinny_bf16_splitk")
    print("  captured kernel", name, flush=True)


def test_decode_fresh_stream_one_split(torch):
    """No scratch on the capturing stream: one split, nothing allocated."""
    case = make_case(16, 4096, 2048, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=82)
    s = torch.cuda.Stream()
    name = capture_and_check(torch, case, s, warm=False, want_prefix="skinny_bf16")
    assert name == "skinny_bf16", name


@pytest.mark.parametrize("tile", ["bf16_pp_256x256x32", "bf16_q4_256x256x32",
                                  "bf16_q16_256x256x32"])
def test_pp_split_shape_unsplit_under_capture(torch, tile, monkeypatch):
    """A shape whose last round would be split runs whole tiles when captured."""
    monkeypatch.setenv("MGEMM_BF16_TILE", tile)
    monkeypatch.setenv("MGEMM_DISABLE_SKINNY", "1")
    case = make_case(1024, 4096, 264, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=83)
    s = torch.cuda.Stream()
    name = capture_and_check(torch, case, s, warm=True, want_prefix=tile)
    assert name == tile, name


def test_fp8_split_shape_unsplit_under_capture(torch):
    """The 8-bit float GEMM: a shape split over K when called directly runs
    whole tiles when captured; every replay (with a direct, split call of the
    same shape between replays) equals the oracle exactly on integers."""
    from roofline_driven_optimisation_amd.inputs import f32_to_fp8_bits
    M, N, K = 1024, 512, 1024
    rng = np.random.default_rng(83)
    a = f32_to_fp8_bits(rng.integers(-4, 5, size=(M, K)).astype(np.float32), 0)
    b = f32_to_fp8_bits(rng.integers(-4, 5, size=(N, K)).astype(np.float32), 0)
    c0 = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    ref, _ = oracle.gemm_fp8(a, b, c0, 1.0, 0.5, 1.0, 1.0, 0)
    A, B = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    C0 = torch.from_numpy(c0).cuda()
    C, D = C0.clone(), C0.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.gemm_fp8(A, B, C, 1.0, 0.5)
    assert binding.last_kernel() == "fp8_q4_256x256x128", binding.last_kernel()
    for r in range(4):
        C.copy_(C0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().astype(np.float64), ref), r
        D.copy_(C0)
        binding.gemm_fp8(A, B, D, 1.0, 0.5)
        assert "splitk" in binding.last_kernel(), binding.last_kernel()
        torch.cuda.synchronize()
        assert np.array_equal(D.cpu().numpy().astype(np.float64), ref), r


@pytest.mark.parametrize("shape", [(70, 300, 520, 72, True), (64, 1024, 128, 136, False)],
                         ids=["qk_persistent", "pv_three_stage"])
def test_batched_under_capture(torch, shape):
    """The batched GEMM's persistent grid (more 256 x 256 tiles than CUs)
    and the three-stage 256 x 128 kernel (tiles that fill every CU) captured
    into a graph: every replay, with eager batched calls of another shape in
    between, equals the oracle exactly on integers."""
    from roofline_driven_optimisation_amd.inputs import f32_to_bf16_bits
    batch, M, N, K, trans_b = shape
    rng = np.random.default_rng(84)
    a = f32_to_bf16_bits(rng.integers(-4, 5, (batch, M, K)).astype(np.float32))
    b = f32_to_bf16_bits(rng.integers(-4, 5, (batch, N, K) if trans_b else (batch, K, N))
                         .astype(np.float32))
    c0 = rng.integers(-8, 9, (batch, M, N)).astype(np.float32)
    ref, _ = oracle.gemm_batched(a, b, c0, 1.0, 0.5, bf16=True, trans_b=trans_b)
    A = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    B = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    C0 = torch.from_numpy(c0).cuda()
    C = C0.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.gemm_bf16_batched(A, B, C, 1.0, 0.5, trans_b=trans_b)
    name = binding.last_kernel()
    assert name.endswith("_persist") if trans_b else "_s3_" in name, name
    oa = torch.ones(3, 264, 64, dtype=torch.bfloat16, device="cuda")
    ob = torch.ones(3, 64, 256, dtype=torch.bfloat16, device="cuda")
    oc = torch.zeros(3, 264, 256, device="cuda")
    for r in range(4):
        C.copy_(C0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().astype(np.float64), ref), (name, r)
        binding.gemm_bf16_batched(oa, ob, oc, 1.0, 0.0)
        torch.cuda.synchronize()
