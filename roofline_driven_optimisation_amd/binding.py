"""Thin ctypes binding over libgemm.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
checks tensor dtypes, shapes, devices and contiguity, then passes raw device
pointers and the HIP stream handle to the C entry points declared in
``include/gemm.h``.  There is no fallback: if the library is missing, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgemm.so"

GEMM_OK = 0
# enum gemm_activation
ACT_NONE, ACT_RELU, ACT_GELU, ACT_SILU = 0, 1, 2, 3
_lock = threading.Lock()
_lib = None


class GemmError(RuntimeError):
    """A non-zero status returned by the C library."""

    def __init__(self, status: int, message: str):
        super().__init__("gemm failed with status %d: %s" % (status, message))
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def library():
    """Load libgemm.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                "%s is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')"
                % path)
        lib = ctypes.CDLL(path)
        i, f, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        for name in ("gemm_f32", "gemm_bf16", "gemm_naive_f32", "gemm_naive_bf16",
                     "gemm_bf16_noalloc"):
            fn = getattr(lib, name)
            fn.argtypes = [i, i, i, f, f, vp, vp, vp, vp]
            fn.restype = ctypes.c_int
        for name in ("gemm_f32_bias_act", "gemm_bf16_bias_act"):
            fn = getattr(lib, name)
            fn.argtypes = [i, i, i, f, f, vp, vp, vp, vp, i, vp]
            fn.restype = ctypes.c_int
        lib.gemm_bf16_strided_batched.argtypes = [i, i, i, i, f, f, vp, ctypes.c_int64, vp,
                                                  ctypes.c_int64, i, vp, ctypes.c_int64, vp]
        lib.gemm_bf16_strided_batched.restype = ctypes.c_int
        lib.gemm_fp8.argtypes = [i, i, i, f, f, vp, vp, vp, f, f, i, vp]
        lib.gemm_fp8.restype = ctypes.c_int
        for name in ("reduce_sum_f32", "reduce_sum_f32_naive"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, ctypes.c_int64, vp, vp]
            fn.restype = ctypes.c_int
        lib.gemm_status_string.argtypes = [ctypes.c_int]
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_last_kernel.argtypes = []
        lib.gemm_last_kernel.restype = ctypes.c_char_p
        lib.gemm_abi_version.argtypes = []
        lib.gemm_abi_version.restype = ctypes.c_int
        lib.gemm_kernel_name.argtypes = [i, i, i, i]
        lib.gemm_kernel_name.restype = ctypes.c_char_p
        lib.gemm_split_timeouts.argtypes = [vp, ctypes.POINTER(ctypes.c_longlong)]
        lib.gemm_split_timeouts.restype = ctypes.c_int
        lib.gemm_test_hook.argtypes = [i, ctypes.c_longlong, vp]
        lib.gemm_test_hook.restype = ctypes.c_int
        lib.gemm_probe_stream.argtypes = [vp, vp, ctypes.c_int64, vp, i, vp]
        lib.gemm_probe_stream.restype = ctypes.c_int
        lib.gemm_probe_lds.argtypes = [i, i, vp, i, vp]
        lib.gemm_probe_lds.restype = ctypes.c_int
        _lib = lib
    return _lib


def _status_message(status: int) -> str:
    return library().gemm_status_string(status).decode()


def last_kernel() -> str:
    """Name of the kernel the last call on this thread launched."""
    return library().gemm_last_kernel().decode()


def kernel_name(dtype: str, M: int, N: int, K: int) -> str:
    """The kernel gemm_bf16 (dtype "bf16") or gemm_f32 ("f32") would launch
    for an M x N x K call on the current device, without launching it."""
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return library().gemm_kernel_name(1 if dtype == "bf16" else 0, int(M), int(N),
                                      int(K)).decode()


# enum gemm_test_hook_id
TEST_POLL_LIMIT, TEST_EPOCH = 1, 2


def split_timeouts(stream=None) -> int:
    """Split-pair waits that gave up on the stream since the last query
    (waits for the stream; clears the count)."""
    count = ctypes.c_longlong(0)
    status = library().gemm_split_timeouts(_stream_handle(stream), ctypes.byref(count))
    if status != GEMM_OK:
        raise GemmError(status, _status_message(status))
    return int(count.value)


def set_test_hook(hook: int, value: int, stream=None) -> None:
    """Set one of the library's test hooks (see gemm_test_hook in gemm.h)."""
    status = library().gemm_test_hook(int(hook), int(value), _stream_handle(stream))
    if status != GEMM_OK:
        raise GemmError(status, _status_message(status))


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(A, B, C, in_dtype):
    import torch
    for name, t in (("A", A), ("B", B), ("C", C)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if t.device.type != "cuda":
            raise ValueError("%s must be on the GPU" % name)
        if t.dim() != 2:
            raise ValueError("%s must be 2-D" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous (packed row-major)" % name)
    if A.dtype != in_dtype or B.dtype != in_dtype:
        raise TypeError("A and B must be %s" % in_dtype)
    if C.dtype != torch.float32:
        raise TypeError("C must be float32")
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on one device")
    M, K = A.shape
    K2, N = B.shape
    if K != K2 or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    return int(M), int(N), int(K)


def _call(fn_name, A, B, C, alpha, beta, stream, in_dtype, epilogue=None):
    import torch
    M, N, K = _check(A, B, C, in_dtype)
    lib = library()
    extra = ()
    if epilogue is not None:
        bias, act = epilogue
        if bias is not None:
            if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32:
                raise TypeError("bias must be a float32 tensor")
            if bias.device != C.device or tuple(bias.shape) != (N,) or not bias.is_contiguous():
                raise ValueError("bias must be a contiguous vector of N = %d on C's device" % N)
        extra = (ctypes.c_void_p(bias.data_ptr() if bias is not None else 0), int(act))
    with torch.cuda.device(C.device):
        status = getattr(lib, fn_name)(M, N, K, float(alpha), float(beta),
                                       ctypes.c_void_p(A.data_ptr()),
                                       ctypes.c_void_p(B.data_ptr()),
                                       ctypes.c_void_p(C.data_ptr()),
                                       *extra, _stream_handle(stream))
    if status != GEMM_OK:
        raise GemmError(status, _status_message(status))
    return C


def gemm_f32(A, B, C, alpha=1.0, beta=0.0, stream=None):
    """C = alpha*A@B + beta*C with float32 A (M x K), B (K x N), C (M x N)."""
    import torch
    return _call("gemm_f32", A, B, C, alpha, beta, stream, torch.float32)


def gemm_bf16(A, B, C, alpha=1.0, beta=0.0, stream=None):
    """C = alpha*A@B + beta*C with bfloat16 A and B, float32 C."""
    import torch
    return _call("gemm_bf16", A, B, C, alpha, beta, stream, torch.bfloat16)


def gemm_bf16_noalloc(A, B, C, alpha=1.0, beta=0.0, stream=None):
    """gemm_bf16 that allocates nothing: its scratch is the library's fixed
    per-GPU array (GemmError with status 5 when the call needs more)."""
    import torch
    return _call("gemm_bf16_noalloc", A, B, C, alpha, beta, stream, torch.bfloat16)


def gemm_f32_bias_act(A, B, C, bias=None, activation=ACT_NONE, alpha=1.0, beta=0.0,
                      stream=None):
    """C = act(alpha*A@B + beta*C + bias) with float32 operands; bias is a
    float32 vector over the N columns or None."""
    import torch
    return _call("gemm_f32_bias_act", A, B, C, alpha, beta, stream, torch.float32,
                 (bias, activation))


def gemm_bf16_bias_act(A, B, C, bias=None, activation=ACT_NONE, alpha=1.0, beta=0.0,
                       stream=None):
    """C = act(alpha*A@B + beta*C + bias) with bfloat16 A and B, float32 C
    and bias."""
    import torch
    return _call("gemm_bf16_bias_act", A, B, C, alpha, beta, stream, torch.bfloat16,
                 (bias, activation))


def gemm_naive_f32(A, B, C, alpha=1.0, beta=0.0, stream=None):
    """The one-thread-per-output kernel (the unoptimised starting point)."""
    import torch
    return _call("gemm_naive_f32", A, B, C, alpha, beta, stream, torch.float32)


def gemm_naive_bf16(A, B, C, alpha=1.0, beta=0.0, stream=None):
    import torch
    return _call("gemm_naive_bf16", A, B, C, alpha, beta, stream, torch.bfloat16)


def gemm_bf16_batched(A, B, C, alpha=1.0, beta=0.0, trans_b=False, stream=None):
    """C[b] = alpha*A[b]@op(B[b]) + beta*C[b] for 3-D contiguous tensors:
    A (batch, M, K) bfloat16, B (batch, K, N) or with trans_b (batch, N, K)
    bfloat16, C (batch, M, N) float32."""
    import torch
    for name, t in (("A", A), ("B", B), ("C", C)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 3-D tensor" % name)
        if t.device.type != "cuda" or t.device != C.device:
            raise ValueError("%s must be on C's GPU" % name)
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16 or C.dtype != torch.float32:
        raise TypeError("A and B must be bfloat16 and C float32")
    batch, M, K = A.shape
    N = B.shape[1] if trans_b else B.shape[2]
    Kb = B.shape[2] if trans_b else B.shape[1]
    if B.shape[0] != batch or Kb != K or tuple(C.shape) != (batch, M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    lib = library()
    with torch.cuda.device(C.device):
        status = lib.gemm_bf16_strided_batched(
            int(batch), int(M), int(N), int(K), float(alpha), float(beta),
            ctypes.c_void_p(A.data_ptr()), M * K, ctypes.c_void_p(B.data_ptr()), K * N,
            1 if trans_b else 0, ctypes.c_void_p(C.data_ptr()), M * N, _stream_handle(stream))
    if status != GEMM_OK:
        raise GemmError(status, _status_message(status))
    return C


FP8_E4M3, FP8_E5M2 = 0, 1


def gemm_fp8(A, B, C, alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0, fmt=FP8_E4M3,
             stream=None):
    """C = alpha*scale_a*scale_b*A@B.T + beta*C with A (M x K) and B (N x K)
    uint8 tensors of 8-bit float bytes (fmt E4M3 or E5M2), C float32."""
    import torch
    for name, t in (("A", A), ("B", B), ("C", C)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 2-D tensor" % name)
        if t.device.type != "cuda" or t.device != C.device:
            raise ValueError("%s must be on C's GPU" % name)
    if A.dtype != torch.uint8 or B.dtype != torch.uint8 or C.dtype != torch.float32:
        raise TypeError("A and B must be uint8 and C float32")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    lib = library()
    with torch.cuda.device(C.device):
        status = lib.gemm_fp8(int(M), int(N), int(K), float(alpha), float(beta),
                              ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                              ctypes.c_void_p(C.data_ptr()), float(scale_a), float(scale_b),
                              int(fmt), _stream_handle(stream))
    if status != GEMM_OK:
        raise GemmError(status, _status_message(status))
    return C


def reduce_sum_f32(x, out, stream=None, naive=False):
    """out[0] = sum of the float32 vector x (both on the GPU; out holds one
    float32).  ``naive`` runs the one-element-per-thread first version."""
    import torch
    for name, t in (("x", x), ("out", out)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
            raise TypeError("%s must be a float32 tensor" % name)
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if out.numel() < 1 or x.device != out.device:
        raise ValueError("out must hold one float on x's device")
    lib = library()
    fn = lib.reduce_sum_f32_naive if naive else lib.reduce_sum_f32
    with torch.cuda.device(x.device):
        status = fn(ctypes.c_void_p(x.data_ptr()), x.numel(), ctypes.c_void_p(out.data_ptr()),
                    _stream_handle(stream))
    if status != GEMM_OK:
        raise GemmError(status, _status_message(status))
    return out


def probe_stream(src, out=None, dst=None, blocks=2048, stream=None):
    """The device bandwidth probe (gemm_probe_stream): read every byte of the
    GPU tensor src once, XOR-folding it into out (uint32 or int32, `blocks`
    words), or copy it into dst when dst is given.  src (and dst) must be
    contiguous, 16-byte aligned, a multiple of 16 bytes long."""
    import torch
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    if dst is not None:
        if (not isinstance(dst, torch.Tensor) or dst.device != src.device or
                not dst.is_contiguous() or dst.numel() * dst.element_size() < nbytes):
            raise ValueError("dst must be a contiguous GPU tensor on src's device, as large")
    if dst is None and (out is None or out.device != src.device or out.element_size() != 4 or
                        not out.is_contiguous() or out.numel() < blocks):
        raise ValueError("out must hold `blocks` 32-bit words on src's device")
    with torch.cuda.device(src.device):
        status = library().gemm_probe_stream(
            ctypes.c_void_p(src.data_ptr()),
            ctypes.c_void_p(dst.data_ptr() if dst is not None else 0), nbytes,
            ctypes.c_void_p(out.data_ptr() if out is not None else 0), int(blocks),
            _stream_handle(stream))
    if status != GEMM_OK:
        raise GemmError(status, _status_message(status))


def probe_lds(stride, steps, out, blocks=512, stream=None):
    """The shared-memory bank probe (gemm_probe_lds): `steps` 4-byte reads
    per lane at lane stride `stride`; out (32-bit words on the GPU, at least
    `blocks`) receives each workgroup's XOR of what it read."""
    import torch
    if out.device.type != "cuda" or out.element_size() != 4 or not out.is_contiguous() or \
            out.numel() < blocks:
        raise ValueError("out must hold `blocks` 32-bit words on the GPU")
    with torch.cuda.device(out.device):
        status = library().gemm_probe_lds(int(stride), int(steps), ctypes.c_void_p(out.data_ptr()),
                                          int(blocks), _stream_handle(stream))
    if status != GEMM_OK:
        raise GemmError(status, _status_message(status))


def gemm(A, B, C, alpha=1.0, beta=0.0, stream=None):
    """Dispatch on A's dtype: float32 -> gemm_f32, bfloat16 -> gemm_bf16."""
    import torch
    if A.dtype == torch.float32:
        return gemm_f32(A, B, C, alpha, beta, stream)
    if A.dtype == torch.bfloat16:
        return gemm_bf16(A, B, C, alpha, beta, stream)
    raise TypeError("unsupported dtype %s" % A.dtype)
