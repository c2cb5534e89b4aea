"""The C-ABI library loads and exports what include/gemm.h declares (no GPU).

Only host-side logic is exercised here: argument validation returns before
any HIP call, and the status/version helpers touch no device.
"""
import ctypes
import os
import re

import pytest

from roofline_driven_optimisation_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"#define GEMM_API.*", "", text)
    return sorted(set(re.findall(r"GEMM_API\s+[\w\s\*]*?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libgemm.so is not built; run __graft_entry__.build() first")
    return binding.library()


def test_header_declares_expected_api():
    names = declared_functions()
    for n in ("gemm_f32", "gemm_bf16", "gemm_naive_f32", "gemm_naive_bf16",
              "gemm_f32_bias_act", "gemm_bf16_bias_act", "reduce_sum_f32", "reduce_sum_f32_naive",
              "gemm_bf16_strided_batched", "gemm_fp8", "gemm_kernel_name",
              "gemm_split_timeouts", "gemm_test_hook", "gemm_probe_stream", "gemm_probe_lds",
              "gemm_status_string", "gemm_last_kernel", "gemm_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_declared_symbols_are_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_abi_version(lib):
    text = open(HEADER).read()
    version = int(re.search(r"#define GEMM_ABI_VERSION (\d+)", text).group(1))
    assert lib.gemm_abi_version() == version


def test_status_strings(lib):
    assert lib.gemm_status_string(0) == b"ok"
    assert lib.gemm_status_string(1) == b"invalid argument"
    assert lib.gemm_status_string(2) == b"kernel launch failed"
    assert lib.gemm_status_string(99) == b"unknown status"


@pytest.mark.parametrize("fn", ["gemm_f32", "gemm_bf16", "gemm_naive_f32", "gemm_naive_bf16"])
def test_validation_without_gpu(lib, fn):
    f = getattr(lib, fn)
    p = ctypes.c_void_p(256)  # never dereferenced: these calls return before any launch
    assert f(-1, 4, 4, 1.0, 0.0, p, p, p, None) == 1
    assert f(4, -1, 4, 1.0, 0.0, p, p, p, None) == 1
    assert f(4, 4, -1, 1.0, 0.0, p, p, p, None) == 1
    assert f(4, 4, 4, 1.0, 0.0, None, p, p, None) == 1   # A missing
    assert f(4, 4, 4, 1.0, 0.0, p, None, p, None) == 1   # B missing
    assert f(4, 4, 4, 1.0, 0.0, p, p, None, None) == 1   # C missing
    # empty outputs are a no-op that launches nothing
    assert f(0, 4, 4, 1.0, 0.0, p, p, None, None) == 0
    assert f(4, 0, 4, 1.0, 0.0, p, None, None, None) == 0
    assert lib.gemm_last_kernel() == b"none"


def test_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    A = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        binding.gemm_f32(A, A, A)  # CPU tensors are refused before any call


def test_kernel_name_without_gpu(lib):
    """The dispatch query answers the cases that need no device: the fp32
    kernel choice depends only on K and N modulo 4, and empty or negative
    shapes are answered before any device query."""
    assert lib.gemm_kernel_name(0, 4096, 4096, 4096) == b"f32_mfma_128x128x32_vec4"
    assert lib.gemm_kernel_name(0, 4092, 4092, 4092) == b"f32_mfma_128x128x32_vec4"
    assert lib.gemm_kernel_name(0, 5, 7, 3) == b"f32_mfma_128x128x32_scalar"
    assert lib.gemm_kernel_name(0, 5, 6, 8) == b"f32_mfma_128x128x32_scalar"
    for is_bf16 in (0, 1):
        assert lib.gemm_kernel_name(is_bf16, 0, 8, 8) == b"none"
        assert lib.gemm_kernel_name(is_bf16, 8, 0, 8) == b"none"
        assert lib.gemm_kernel_name(is_bf16, 8, 8, 0) == b"scale_c"
        assert lib.gemm_kernel_name(is_bf16, -1, 8, 8) == b"invalid"
        assert lib.gemm_kernel_name(is_bf16, 8, 8, -1) == b"invalid"


def test_diagnostics_argument_errors(lib):
    assert lib.gemm_split_timeouts(None, None) == 1
    assert lib.gemm_test_hook(99, 0, None) == 1


def test_probe_argument_errors(lib):
    """The probes' argument checks return before any HIP call."""
    p = ctypes.c_void_p(256)  # never dereferenced
    u = ctypes.c_void_p(260)  # not 16-byte aligned
    assert lib.gemm_probe_stream(p, None, -16, p, 1, None) == 1        # negative size
    assert lib.gemm_probe_stream(p, None, 24, p, 1, None) == 1         # not a multiple of 16
    assert lib.gemm_probe_stream(u, None, 32, p, 1, None) == 1         # misaligned src
    assert lib.gemm_probe_stream(p, u, 32, None, 1, None) == 1         # misaligned dst
    assert lib.gemm_probe_stream(None, None, 32, p, 1, None) == 1      # no src
    assert lib.gemm_probe_stream(p, None, 32, None, 1, None) == 1      # read with no out
    assert lib.gemm_probe_stream(p, None, 32, p, 0, None) == 1         # no workgroups
    assert lib.gemm_probe_stream(p, None, 32, p, (1 << 20) + 1, None) == 1
    assert lib.gemm_probe_lds(1, 8, None, 1, None) == 1                # no out
    assert lib.gemm_probe_lds(-1, 8, p, 1, None) == 1
    assert lib.gemm_probe_lds(1, -1, p, 1, None) == 1
    assert lib.gemm_probe_lds(1, 8, p, 0, None) == 1
    assert lib.gemm_probe_lds(64, 16384 - 63 * 64 - 51 + 1, p, 1, None) == 1  # past the table
    assert lib.gemm_probe_lds(300, 8, p, 1, None) == 1               # lanes past the table
    assert lib.gemm_last_kernel() == b"none"
