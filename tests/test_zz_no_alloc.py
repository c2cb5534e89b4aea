"""gemm_bf16_noalloc, the entry point that allocates nothing, through the C
ABI against gemm_bf16 on the same seeded inputs.

* Decode-shaped calls (the path whose kernel uses the static scratch), two
  in a row, the second smaller: equal to gemm_bf16's output bit for bit on
  integer inputs, and within the bf16 tolerance of the oracle (and of
  gemm_bf16) on random ones.
* A large-M call runs whole tiles and matches gemm_bf16.
* A decode-shaped call that needs more scratch than the array holds is
  refused with GEMM_ERR_SCRATCH and leaves C untouched.
* Under graph capture (on a stream with no workspace) the decode call still
  splits K through the static array, and every replay is exact.
* In a fresh child process (where the first call sets the array up and
  runs the XCD probe itself): once every shape has run, further calls of
  all of them leave the device's free memory unchanged.
"""
import ctypes
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, log, to_device
from roofline_driven_optimisation_amd import binding
from roofline_driven_optimisation_amd.inputs import make_case

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_ERR_SCRATCH = 5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.library()
    oracle.build(force=False)
    return torch


def call(name, case, c_fill=np.nan):
    """(status, kernel, C) of one C-ABI call on the current stream."""
    import torch
    lib = binding.library()
    A, B, C = to_device(case, c_fill)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    log("  %s %dx%dx%d" % (name, case.M, case.N, case.K))
    rc = getattr(lib, name)(case.M, case.N, case.K, case.alpha, case.beta,
                            ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                            ctypes.c_void_p(C.data_ptr()), s)
    kernel = binding.last_kernel()
    torch.cuda.synchronize()
    return rc, kernel, C.cpu().numpy()


SEQUENCE = [(16, 11008, 4096), (8, 4096, 4096)]  # the second call is smaller


def test_noalloc_decode_integer_exact():
    for shape in SEQUENCE:
        case = make_case(*shape, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=61)
        rc0, k0, C0 = call("gemm_bf16", case)
        rc1, k1, C1 = call("gemm_bf16_noalloc", case)
        assert rc0 == 0 and rc1 == 0, (rc0, rc1)
        assert k1 == "skinny_bf16_splitk_xcd_static", k1
        assert np.array_equal(C1, C0), shape
        ref, _ = oracle.gemm(case.A, case.B, case.C, 1.5, 0.5, bf16=True)
        assert np.array_equal(C1.astype(np.float64), ref), shape


def test_noalloc_decode_random():
    for shape in SEQUENCE:
        case = make_case(*shape, "bf16", 1.0, 0.0, "n:1", "n:0.02", seed=62)
        _, _, C0 = call("gemm_bf16", case)
        rc, k1, C1 = call("gemm_bf16_noalloc", case)
        assert rc == 0 and k1 == "skinny_bf16_splitk_xcd_static", (rc, k1)
        ref, den = oracle.gemm(case.A, case.B, None, 1.0, 0.0, bf16=True)
        err_oracle = oracle.parity_error(C1, ref, den)
        err_pair = oracle.parity_error(C1, C0.astype(np.float64), den)
        log("  noalloc %s: err vs oracle %.3e, vs gemm_bf16 %.3e" % (shape, err_oracle, err_pair))
        assert err_oracle <= TOL["bf16"] and err_pair <= TOL["bf16"]


def test_noalloc_tiled_whole_tiles():
    case = make_case(512, 1024, 512, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=63)
    _, k0, C0 = call("gemm_bf16", case)
    rc, k1, C1 = call("gemm_bf16_noalloc", case)
    assert rc == 0 and "splitk" not in k1, (rc, k1)
    assert np.array_equal(C1, C0)


def test_noalloc_refuses_oversized():
    case = make_case(16, 16384, 4096, "bf16", 1.0, 0.0, "i:4", "i:4", seed=64)
    rc, k, C = call("gemm_bf16_noalloc", case, c_fill=7.0)
    assert rc == GEMM_ERR_SCRATCH and k == "none", (rc, k)
    assert np.all(C == 7.0)
    assert binding.library().gemm_status_string(rc).decode().startswith("the call needs more")


def test_noalloc_under_graph_capture():
    """The callers it is for include code under HIP graph capture: after one
    direct call has set the array up, a decode-shaped call captured on a
    fresh stream (which has no workspace of its own) splits K through the
    static array, and four replays, with eager calls of both entry points
    on another shape between them, each give the oracle's result exactly
    (the kernel re-arms its counters, so every replay starts clean)."""
    import torch
    case = make_case(16, 4096, 2048, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=65)
    ref, _ = oracle.gemm(case.A, case.B, case.C, 1.5, 0.5, bf16=True)
    A, B, C = to_device(case)
    C0 = C.clone()
    rc, k, _ = call("gemm_bf16_noalloc", case)  # set-up on this device (if not done yet)
    assert rc == 0 and k == "skinny_bf16_splitk_xcd_static", (rc, k)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.gemm_bf16_noalloc(A, B, C, 1.5, 0.5)
    assert binding.last_kernel() == "skinny_bf16_splitk_xcd_static", binding.last_kernel()
    other = make_case(8, 1024, 512, "bf16", 1.0, 0.0, "i:4", "i:4", seed=66)
    oA, oB, oC = to_device(other)
    for r in range(4):
        C.copy_(C0)
        g.replay()
        torch.cuda.synchronize()
        log("  graph replay %d" % r)
        assert np.array_equal(C.cpu().numpy().astype(np.float64), ref), r
        binding.gemm_bf16_noalloc(oA, oB, oC, 1.0, 0.0)
        binding.gemm_bf16(oA, oB, oC, 1.0, 0.0)
        torch.cuda.synchronize()


def test_noalloc_fresh_process_allocates_nothing():
    env = dict(os.environ)
    env.setdefault("HSA_ENABLE_IPC_MODE_LEGACY", "0")
    log("  child: no-allocation entry point in a fresh process")
    r = subprocess.run([sys.executable, os.path.join(HERE, "no_alloc_child.py")],
                       capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.returncode
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["kernels"][0] == "skinny_bf16_splitk_xcd_static", out
    assert out["exact"] == [True] * len(out["exact"]), out
    assert out["free_before_later_rounds"] == out["free_after_later_rounds"], out
