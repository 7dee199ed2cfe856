"""Python binding of the q4 C library (libq4.so): group-wise INT4 RTN quantization and the
W4A16 matmul on AMD MI355X.

Argument marshalling only: every step runs in the library's HIP kernels.  torch is used for
device memory and the current stream.  The functions raise Q4Error (a ValueError) carrying
the library's status string; they raise RuntimeError if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "Q4Error", "library", "library_path", "quantize_rtn", "quantize_rtn_into", "matmul",
    "matmul_into", "dequantize", "dequantize_into", "select_kernel", "status_string", "version",
    "MODES", "KERNELS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libq4.so")

MODES = {"asym": 0, "sym": 1}
KERNELS = {"auto": 0, "gemv": 1, "gemm": 2, "decode": 3}
_KERNEL_NAMES = {v: k for k, v in KERNELS.items()}

_lock = threading.Lock()
_lib = None


class Q4Error(ValueError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library() -> ctypes.CDLL:
    """Load libq4.so (once).  There is no fallback: a missing library is an error."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(library_path):
                raise RuntimeError(f"{library_path} is not built; run "
                                   "`python -m weight_only_int4_group_amd.build`")
            lib = ctypes.CDLL(library_path)
            i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
            lib.q4_quantize_rtn.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
            lib.q4_quantize_rtn.restype = ctypes.c_int
            lib.q4_matmul.argtypes = [vp, i64, i64, i64, i32, i32, vp, vp, vp, vp, vp]
            lib.q4_matmul.restype = ctypes.c_int
            lib.q4_matmul_kernel.argtypes = [vp, i64, i64, i64, i32, i32, vp, vp, vp, vp, i32, vp]
            lib.q4_matmul_kernel.restype = ctypes.c_int
            lib.q4_dequantize.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, i32, vp]
            lib.q4_dequantize.restype = ctypes.c_int
            lib.q4_select_kernel.argtypes = [i64, i64, i64, i32]
            lib.q4_select_kernel.restype = ctypes.c_int
            lib.q4_status_string.argtypes = [ctypes.c_int]
            lib.q4_status_string.restype = ctypes.c_char_p
            lib.q4_version.argtypes = []
            lib.q4_version.restype = ctypes.c_int
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().q4_status_string(int(status)).decode()


def version() -> int:
    return int(library().q4_version())


def select_kernel(M: int, N: int, K: int, g: int) -> str:
    st = library().q4_select_kernel(M, N, K, g)
    if st < 0:
        raise Q4Error(st, "q4_select_kernel")
    return _KERNEL_NAMES[st]


def _mode(mode: str) -> int:
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}, got {mode!r}")
    return MODES[mode]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def quantize_rtn_into(W, g: int, mode: str, packed, scales, zeros) -> None:
    """q4_quantize_rtn on caller-provided outputs (no allocation)."""
    import torch
    _check_cuda(W, packed, scales, zeros)
    if W.dtype != torch.bfloat16 or W.dim() != 2:
        raise ValueError("W must be a 2-D bfloat16 tensor")
    N, K = W.shape
    with torch.cuda.device(W.device):
        st = library().q4_quantize_rtn(_ptr(W), N, K, g, _mode(mode), _ptr(packed), _ptr(scales),
                                       _ptr(zeros), _stream(W.device))
    if st != 0:
        raise Q4Error(st, "q4_quantize_rtn")


def quantize_rtn(W, g: int = 128, mode: str = "asym"):
    """W[N, K] bf16 -> (packed uint8[N, K/2], scales fp16[N, K/g], zeros uint8[N, K/g])."""
    import torch
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    G = K // g if g > 0 else 0
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=W.device)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=W.device)
    quantize_rtn_into(W, g, mode, packed, scales, zeros)
    return packed, scales, zeros


def matmul_into(X, packed, scales, zeros, g: int, mode: str, Y, kernel: str = "auto") -> None:
    """q4_matmul_kernel on a caller-provided Y (no allocation)."""
    import torch
    _check_cuda(X, packed, scales, zeros, Y)
    if X.dtype != torch.bfloat16 or X.dim() != 2 or Y.dtype != torch.bfloat16:
        raise ValueError("X and Y must be 2-D bfloat16 tensors")
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    M, K = X.shape
    N = packed.shape[0]
    if packed.shape[1] * 2 != K or tuple(Y.shape) != (M, N):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, packed {tuple(packed.shape)}, Y {tuple(Y.shape)}")
    with torch.cuda.device(packed.device):
        st = library().q4_matmul_kernel(_ptr(X), M, N, K, g, _mode(mode), _ptr(packed),
                                        _ptr(scales), _ptr(zeros), _ptr(Y), KERNELS[kernel],
                                        _stream(packed.device))
    if st != 0:
        raise Q4Error(st, "q4_matmul")


def matmul(X, packed, scales, zeros, g: int = 128, mode: str = "asym", kernel: str = "auto"):
    """Y[M, N] = X[M, K] @ dequant(packed, scales, zeros)^T, bf16."""
    import torch
    Y = torch.empty((X.shape[0], packed.shape[0]), dtype=torch.bfloat16, device=packed.device)
    matmul_into(X, packed, scales, zeros, g, mode, Y, kernel)
    return Y


def _out_dtype(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return 0
    if dtype == torch.float16:
        return 1
    raise ValueError(f"out dtype must be bfloat16 or float16, got {dtype}")


def dequantize_into(packed, scales, zeros, g: int, mode: str, out) -> None:
    """q4_dequantize on a caller-provided out[N, K] (bfloat16 or float16; no allocation)."""
    _check_cuda(packed, scales, zeros, out)
    if packed.dim() != 2:
        raise ValueError("packed must be 2-D")
    N, K = packed.shape[0], packed.shape[1] * 2
    if tuple(out.shape) != (N, K):
        raise ValueError(f"shape mismatch: packed {tuple(packed.shape)}, out {tuple(out.shape)}")
    with __import__("torch").cuda.device(packed.device):
        st = library().q4_dequantize(N, K, g, _mode(mode), _ptr(packed), _ptr(scales), _ptr(zeros),
                                     _ptr(out), _out_dtype(out.dtype), _stream(packed.device))
    if st != 0:
        raise Q4Error(st, "q4_dequantize")


def dequantize(packed, scales, zeros, g: int = 128, mode: str = "asym", dtype=None):
    """dequant(packed, scales, zeros) as an [N, K] tensor (bfloat16 unless dtype says float16)."""
    import torch
    out = torch.empty((packed.shape[0], packed.shape[1] * 2),
                      dtype=torch.bfloat16 if dtype is None else dtype, device=packed.device)
    dequantize_into(packed, scales, zeros, g, mode, out)
    return out
