"""The split pairs' handshake and the per-stream workspaces, through the C ABI.

* A wait that gives up is counted and can be read back with
  gemm_split_timeouts; the give-up is forced from the host (the poll-limit
  test hook set to zero), so every kernel still runs to its end.
* The 32-bit split epoch wraps to 1 without reusing a flag or claim word
  left from an earlier call (the library clears them first).
* Streams beyond the library's workspace cap run the same kernels without
  splitting K and give the same results (in a child process, so that the
  cap is not used up for the other tests).

Integer inputs in [-4, 4] make every partial sum exact in fp32, so results
are compared with the oracle bit for bit.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from gpu_helpers import log, run, to_device
from roofline_driven_optimisation_amd import binding
from roofline_driven_optimisation_amd.inputs import make_case

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))

# (M, N, K, kernel): every tile of these shapes is split over K (fewer tiles
# than half the CUs); one tile pairs workgroups on two XCDs, eight tiles pair
# them on one XCD.
SPLIT = [(256, 256, 512, "bf16_q4_256x256x32_splitk"),
         (512, 1024, 512, "bf16_q4_256x256x32_splitk_xcd")]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.library()
    oracle.build(force=False)
    return torch


def exact(case, C):
    ref, _ = oracle.gemm(case.A, case.B, case.C, case.alpha, case.beta, bf16=case.bf16)
    return np.array_equal(C.astype(np.float64), ref)


@pytest.fixture
def q4(monkeypatch):
    """The four-wave 256 x 256 kernel for every tiled call (at these small
    shapes the tile picker would take smaller tiles, which never split)."""
    monkeypatch.setenv("MGEMM_BF16_TILE", "bf16_q4_256x256x32")


@pytest.mark.parametrize("shape", SPLIT, ids=["pairs", "xcd"])
def test_split_wait_timeout_is_reported(shape, q4):
    M, N, K, want = shape
    case = make_case(M, N, K, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=41)
    tiles = (M // 256) * (N // 256)
    binding.split_timeouts()  # start from zero
    try:
        binding.set_test_hook(binding.TEST_POLL_LIMIT, 0)
        C, name = run(case)
        assert name == want, name
        given_up = binding.split_timeouts()
        log("  poll limit 0: %d waits gave up, %d split tiles" % (given_up, tiles))
        assert given_up == tiles
        assert np.isnan(C).all()  # each wait that gave up marks its tile
    finally:
        binding.set_test_hook(binding.TEST_POLL_LIMIT, -1)
    C, name = run(case)
    assert name == want, name
    assert binding.split_timeouts() == 0
    assert exact(case, C)


def test_fp8_split_wait_timeout_is_reported(gpu):
    torch = gpu
    from roofline_driven_optimisation_amd.inputs import f32_to_fp8_bits
    M, N, K = 520, 300, 1072  # 3 x 2 tiles, all split, pairs on two XCDs
    rng = np.random.default_rng(42)
    A = f32_to_fp8_bits(rng.integers(-4, 5, (M, K)).astype(np.float32), 0)
    B = f32_to_fp8_bits(rng.integers(-4, 5, (N, K)).astype(np.float32), 0)
    At, Bt = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    binding.split_timeouts()
    try:
        binding.set_test_hook(binding.TEST_POLL_LIMIT, 0)
        Ct = torch.zeros(M, N, device="cuda")
        binding.gemm_fp8(At, Bt, Ct, 1.0, 0.0)
        assert binding.last_kernel() == "fp8_q4_256x256x128_splitk"
        assert binding.split_timeouts() == 6
        assert bool(torch.isnan(Ct).all())
    finally:
        binding.set_test_hook(binding.TEST_POLL_LIMIT, -1)
    Ct = torch.zeros(M, N, device="cuda")
    binding.gemm_fp8(At, Bt, Ct, 1.0, 0.0)
    assert binding.split_timeouts() == 0
    ref, _ = oracle.gemm_fp8(A, B, None, 1.0, 0.0, 1.0, 1.0, 0)
    assert np.array_equal(Ct.cpu().numpy().astype(np.float64), ref)


def test_split_epoch_wrap(q4):
    """Calls on both pair forms across the point where the epoch wraps.  The
    pre-wrap calls leave epochs 1 (uncached block) and 2 (XCD-local block)
    in the flag and claim words that the first post-wrap calls take again,
    with different inputs: without the clearing at the wrap, both workgroups
    of a pair would take the stale words for their partner's and add a
    stale partial tile."""
    a, b = SPLIT
    mk = lambda s, seed: make_case(s[0], s[1], s[2], "bf16", 1.5, 0.5, "i:4", "i:4", "i:4",
                                   seed=seed)
    C, _ = run(mk(a, 50))  # the stream's workspace exists from here on
    binding.set_test_hook(binding.TEST_EPOCH, 0)
    before = [(a, 51), (b, 52)]                  # epochs 1, 2
    after = [(a, 53), (b, 54), (a, 55), (b, 56)]  # 2^32 wraps to 0: cleared, then 1, 2, 3, 4
    for shape, seed in before:
        case = mk(shape, seed)
        C, name = run(case)
        assert name == shape[3], name
        assert exact(case, C), (shape, seed)
    binding.set_test_hook(binding.TEST_EPOCH, 2 ** 32 - 1)
    for shape, seed in after:
        case = mk(shape, seed)
        C, name = run(case)
        log("  after the wrap: %s seed %d" % (name, seed))
        assert name == shape[3], name
        assert exact(case, C), (shape, seed)
    assert binding.split_timeouts() == 0


def test_workspace_cap_in_child():
    """Twenty streams in a fresh process: the first sixteen get a workspace
    and split K, the others run the decode GEMM in one split; all exact."""
    env = dict(os.environ)
    env.setdefault("HSA_ENABLE_IPC_MODE_LEGACY", "0")
    log("  child: workspace cap")
    r = subprocess.run([sys.executable, os.path.join(HERE, "workspace_cap_child.py")],
                       capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.returncode
    out = json.loads(r.stdout.strip().splitlines()[-1])
    names = out["names"]
    assert len(names) == 20
    assert all(n == "skinny_bf16_splitk_xcd" for n in names[:16]), names
    assert all(n == "skinny_bf16" for n in names[16:]), names
    assert out["exact"] == [True] * 20
