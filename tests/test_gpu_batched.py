"""GPU parity of the strided batched bf16 GEMM (attention's S = Q K^T with K
stored token-major, and O = P V) through the C ABI, against the oracle item
by item: every path (the four-wave 256 x 256 kernel with B as K x N or
stored transposed, on one workgroup per tile or on a persistent grid when
there are more tiles than CUs, the 128 x 128 kernel for N <= 128 and,
forced, with B stored transposed, C through LDS or straight from the
accumulators, the one-thread-per-output fallback), exact on integer
inputs, within the bf16 tolerance on random ones, and at the attention
shapes of a 2048-token, 32-head, d = 128 layer over every head's whole
output."""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, log
from roofline_driven_optimisation_amd import binding
from roofline_driven_optimisation_amd.inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def widen(bits):
    """bf16 bit patterns to their exact values (the upper half of an fp32)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def draw(shape, dist, rng):
    if dist.startswith("i:"):
        r = int(dist[2:])
        return rng.integers(-r, r + 1, size=shape).astype(np.float32)
    return (rng.standard_normal(size=shape) * float(dist[2:])).astype(np.float32)


def make(batch, M, N, K, trans_b, dist_a, dist_b, beta, seed):
    rng = np.random.default_rng(seed)
    A = f32_to_bf16_bits(draw((batch, M, K), dist_a, rng))
    B = f32_to_bf16_bits(draw((batch, N, K) if trans_b else (batch, K, N), dist_b, rng))
    C = draw((batch, M, N), "i:4", rng) if beta != 0.0 else None
    return A, B, C


def run(A, B, C, alpha, beta, trans_b, N):
    import torch
    batch, M, K = A.shape
    At = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).cuda()
    Bt = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).cuda()
    Ct = (torch.from_numpy(C).cuda() if C is not None
          else torch.full((batch, M, N), float("nan"), device="cuda"))
    log("  gpu batched %dx%dx%dx%d trans_b=%s beta=%g" % (batch, M, N, K, trans_b, beta))
    binding.gemm_bf16_batched(At, Bt, Ct, alpha, beta, trans_b=trans_b)
    name = binding.last_kernel()
    torch.cuda.synchronize()
    return Ct.cpu().numpy(), name


CASES = [  # (batch, M, N, K, trans_b, expected kernel)
    (3, 300, 520, 128, True, "bf16_q4_256x256x32_batched_bt"),
    (3, 300, 520, 136, True, "bf16_q4_256x256x32_batched_bt"),   # K tail
    (3, 300, 520, 136, False, "bf16_q4_256x256x32_batched"),
    (4, 300, 128, 264, False, "bf16_mfma_128x128x64_batched"),
    (2, 264, 120, 72, False, "bf16_mfma_128x128x64_batched"),   # N < 128
    (1, 512, 512, 64, True, "bf16_q4_256x256x32_batched_bt"),
    (3, 37, 100, 60, False, "naive_bf16_batched"),
    (3, 37, 100, 60, True, "naive_bf16_batched"),
    (2, 70, 130, 64, True, "naive_bf16_batched"),                # N % 8 != 0, B transposed
    (2, 40, 72, 0, True, "naive_bf16_batched"),                  # K = 0: beta * C
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%dx%d_%s" % (c[:4] + ("bt" if c[4] else "bn",)))
def test_batched_exact_integers(case):
    batch, M, N, K, trans_b, want = case
    A, B, C = make(batch, M, N, K, trans_b, "i:4", "i:4", 0.5, seed=batch * 100 + K)
    got, name = run(A, B, C, 1.0, 0.5, trans_b, N)
    assert name == want, name
    ref, _ = oracle.gemm_batched(A, B, C, 1.0, 0.5, bf16=True, trans_b=trans_b)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("case", CASES[:6], ids=lambda c: "%dx%dx%dx%d_%s" % (c[:4] + ("bt" if c[4] else "bn",)))
def test_batched_random(case):
    batch, M, N, K, trans_b, want = case
    A, B, C = make(batch, M, N, K, trans_b, "n:1", "n:0.1", 0.0, seed=7 + K)
    got, name = run(A, B, None, 1.25, 0.0, trans_b, N)
    ref, den = oracle.gemm_batched(A, B, None, 1.25, 0.0, bf16=True, trans_b=trans_b)
    err = oracle.parity_error(got, ref, den)
    log("  batched parity err=%.3e" % err)
    assert err <= TOL["bf16"]


# the 128 x 128 tile forced (MGEMM_BF16_TILE), B either way, C stored
# through LDS (the default) or straight from the accumulators
# (MGEMM_BATCHED_STAGED=0)
TILE128 = [  # (batch, M, N, K, trans_b)
    (3, 300, 520, 128, True),
    (3, 300, 520, 136, True),    # K tail
    (2, 264, 120, 72, True),     # N < 128, two K steps with a tail
    (1, 512, 512, 64, True),
    (3, 300, 520, 136, False),
    (4, 300, 128, 264, False),
]


def force_128(monkeypatch, staged):
    monkeypatch.setenv("MGEMM_BF16_TILE", "bf16_mfma_128x128x64")
    monkeypatch.setenv("MGEMM_BATCHED_STAGED", "1" if staged else "0")


def name_128(trans_b, staged):
    return ("bf16_mfma_128x128x64_batched" + ("_bt" if trans_b else "") +
            ("" if staged else "_direct"))


@pytest.mark.parametrize("staged", [False, True], ids=["direct", "lds"])
@pytest.mark.parametrize("case", TILE128, ids=lambda c: "%dx%dx%dx%d_%s" % (c[:4] + ("bt" if c[4] else "bn",)))
def test_batched_128_tile(case, staged, monkeypatch):
    """Exact on integers (beta 0.5) and within the bf16 tolerance on normal
    draws."""
    batch, M, N, K, trans_b = case
    force_128(monkeypatch, staged)
    A, B, C = make(batch, M, N, K, trans_b, "i:4", "i:4", 0.5, seed=batch * 100 + K + 1)
    got, name = run(A, B, C, 1.0, 0.5, trans_b, N)
    assert name == name_128(trans_b, staged), name
    ref, _ = oracle.gemm_batched(A, B, C, 1.0, 0.5, bf16=True, trans_b=trans_b)
    assert np.array_equal(got.astype(np.float64), ref)
    A, B, _ = make(batch, M, N, K, trans_b, "n:1", "n:0.1", 0.0, seed=8 + K)
    got, _ = run(A, B, None, 1.25, 0.0, trans_b, N)
    ref, den = oracle.gemm_batched(A, B, None, 1.25, 0.0, bf16=True, trans_b=trans_b)
    assert oracle.parity_error(got, ref, den) <= TOL["bf16"]


# O = P V shapes (N <= 128, B as K x N) on deeper pipelines
# (MGEMM_BATCHED_DEEP): 128 x 128 tiles on four LDS stages (1) and 256 x 128
# tiles on three (2), copies up to three K steps ahead, C either way.
DEEP = [  # (batch, M, N, K)
    (4, 300, 128, 264),    # five K steps, the last a tail
    (2, 264, 120, 72),     # N < 128, fewer K steps than stages
    (3, 520, 128, 64),     # one K step
    (5, 256, 128, 1000),   # 16 K steps, a tail
]


@pytest.mark.parametrize("staged", [False, True], ids=["direct", "lds"])
@pytest.mark.parametrize("deep", [1, 2])
@pytest.mark.parametrize("case", DEEP, ids=lambda c: "%dx%dx%dx%d" % c)
def test_batched_deep(case, deep, staged, monkeypatch):
    batch, M, N, K = case
    monkeypatch.setenv("MGEMM_BATCHED_DEEP", str(deep))
    monkeypatch.setenv("MGEMM_BATCHED_STAGED", "1" if staged else "0")
    A, B, C = make(batch, M, N, K, False, "i:4", "i:4", 0.5, seed=batch * 100 + K + 3)
    got, name = run(A, B, C, 1.0, 0.5, False, N)
    want = ("bf16_mfma_128x128x64_s4_batched" if deep == 1 else
            "bf16_mfma_256x128x64_s3_batched") + ("" if staged else "_direct")
    assert name == want, name
    ref, _ = oracle.gemm_batched(A, B, C, 1.0, 0.5, bf16=True)
    assert np.array_equal(got.astype(np.float64), ref)
    A, B, _ = make(batch, M, N, K, False, "n:1", "n:0.1", 0.0, seed=10 + K)
    got, _ = run(A, B, None, 1.25, 0.0, False, N)
    ref, den = oracle.gemm_batched(A, B, None, 1.25, 0.0, bf16=True)
    assert oracle.parity_error(got, ref, den) <= TOL["bf16"]


# More 256 x 256 tiles than CUs: the persistent grid, whose workgroups take
# every 256th tile and copy the next tile's first K steps while storing C.
PERSIST = [  # (batch, M, N, K, trans_b)
    (70, 300, 520, 72, True),     # 420 tiles, K tail, ragged M and N
    (70, 300, 520, 128, False),
    (70, 300, 520, 32, True),     # one K step per tile
    (70, 300, 520, 64, False),    # two K steps per tile
    (130, 256, 512, 96, True),    # 260 tiles: four workgroups take two tiles
    (80, 264, 264, 200, False),   # 320 tiles, K tail
]


@pytest.mark.parametrize("case", PERSIST, ids=lambda c: "%dx%dx%dx%d_%s" % (c[:4] + ("bt" if c[4] else "bn",)))
def test_batched_persistent(case, monkeypatch):
    """Exact on integers with beta 0.5 (C read back in every tile's
    epilogue), and on normal draws bit-identical to one workgroup per tile
    (MGEMM_BATCHED_PERSIST=0): each tile's sums are formed in the same order
    either way."""
    batch, M, N, K, trans_b = case
    A, B, C = make(batch, M, N, K, trans_b, "i:4", "i:4", 0.5, seed=batch * 100 + K + 2)
    got, name = run(A, B, C, 1.0, 0.5, trans_b, N)
    assert name == "bf16_q4_256x256x32_batched" + ("_bt" if trans_b else "") + "_persist", name
    ref, _ = oracle.gemm_batched(A, B, C, 1.0, 0.5, bf16=True, trans_b=trans_b)
    assert np.array_equal(got.astype(np.float64), ref)
    A, B, _ = make(batch, M, N, K, trans_b, "n:1", "n:0.1", 0.0, seed=9 + K)
    got, _ = run(A, B, None, 1.25, 0.0, trans_b, N)
    ref, den = oracle.gemm_batched(A, B, None, 1.25, 0.0, bf16=True, trans_b=trans_b)
    assert oracle.parity_error(got, ref, den) <= TOL["bf16"]
    monkeypatch.setenv("MGEMM_BATCHED_PERSIST", "0")
    one, name = run(A, B, None, 1.25, 0.0, trans_b, N)
    assert name == "bf16_q4_256x256x32_batched" + ("_bt" if trans_b else ""), name
    assert np.array_equal(got.view(np.uint32), one.view(np.uint32))


@pytest.mark.parametrize("trans_b", [True, False], ids=["qk", "pv"])
def test_attention_shapes_full(trans_b):
    """32 heads, 2048 tokens, d = 128: S = Q K^T (M = N = 2048, K = 128, K
    stored token-major) and O = P V (M = 2048, N = 128, K = 2048), every
    head's whole output against the oracle."""
    H, T, d = 32, 2048, 128
    M, N, K = (T, T, d) if trans_b else (T, d, T)
    rng = np.random.default_rng(3)
    A = f32_to_bf16_bits(draw((H, M, K), "n:1", rng))
    B = f32_to_bf16_bits(draw((H, N, K) if trans_b else (H, K, N), "n:0.1", rng))
    got, name = run(A, B, None, 1.0, 0.0, trans_b, N)
    assert name.startswith("bf16_"), name
    worst = 0.0
    for h in range(H):
        Bh = np.ascontiguousarray(B[h].T) if trans_b else B[h]
        ref, den = oracle.gemm(A[h], Bh, bf16=True)
        worst = max(worst, oracle.parity_error(got[h], ref, den))
    log("  attention %s, all %d heads, err=%.3e" % ("qk" if trans_b else "pv", H, worst))
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("tile", ["picked", "128_direct", "128_lds"])
@pytest.mark.parametrize("trans_b", [True, False], ids=["qk", "pv"])
def test_attention_shapes_integers(trans_b, tile, monkeypatch):
    """The same 32-head shapes with integer entries in [-3, 3]: every partial
    sum is an integer below 2^24, so all 32 heads' outputs must equal the
    exact products bit for bit (with the tile the library picks, and with
    the 128 x 128 tile either way of storing C)."""
    if tile != "picked":
        force_128(monkeypatch, tile == "128_lds")
    H, T, d = 32, 2048, 128
    M, N, K = (T, T, d) if trans_b else (T, d, T)
    rng = np.random.default_rng(4)
    A = f32_to_bf16_bits(rng.integers(-3, 4, (H, M, K)).astype(np.float32))
    Bs = (H, N, K) if trans_b else (H, K, N)
    B = f32_to_bf16_bits(rng.integers(-3, 4, Bs).astype(np.float32))
    got, name = run(A, B, None, 1.0, 0.0, trans_b, N)
    assert name.startswith("bf16_"), name
    a = widen(A)
    b = widen(B)
    ref = a @ (np.swapaxes(b, 1, 2) if trans_b else b)
    assert np.array_equal(got.astype(np.float64), ref)


def test_shared_operand_stride_zero():
    """stride_b = 0: every item multiplies by the same B."""
    import torch
    lib = binding.library()
    rng = np.random.default_rng(9)
    batch, M, N, K = 3, 264, 256, 64
    A = f32_to_bf16_bits(draw((batch, M, K), "i:3", rng))
    B = f32_to_bf16_bits(draw((K, N), "i:3", rng))
    At = torch.from_numpy(A.view(np.int16)).cuda()
    Bt = torch.from_numpy(B.view(np.int16)).cuda()
    Ct = torch.zeros(batch, M, N, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.gemm_bf16_strided_batched(batch, M, N, K, 1.0, 0.0, ctypes.c_void_p(At.data_ptr()),
                                       M * K, ctypes.c_void_p(Bt.data_ptr()), 0, 0,
                                       ctypes.c_void_p(Ct.data_ptr()), M * N, s)
    assert rc == 0
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_batched(A, np.stack([B] * batch), bf16=True)
    assert np.array_equal(Ct.cpu().numpy().astype(np.float64), ref)


def test_batched_bad_arguments():
    import torch
    lib = binding.library()
    x = torch.zeros(4096, dtype=torch.int16, device="cuda")
    c = torch.zeros(4096, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    args = lambda batch, tb, sc: (batch, 8, 8, 8, 1.0, 0.0, p(x), 64, p(x), 64, tb, p(c), sc, s)
    assert lib.gemm_bf16_strided_batched(*args(-1, 0, 64)) == 1
    assert lib.gemm_bf16_strided_batched(*args(2, 2, 64)) == 1
    assert lib.gemm_bf16_strided_batched(*args(2, 0, 32)) == 1   # items would overlap in C
    assert lib.gemm_bf16_strided_batched(*args(0, 0, 64)) == 0   # nothing to do
    torch.cuda.synchronize()
