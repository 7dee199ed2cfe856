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
    "matmul_into", "dequantize", "dequantize_into", "quantize_rtn_scaled", "quantize_rtn_scaled_into",
    "scale_columns", "scale_columns_into", "awq_workspace_bytes", "awq_search", "awq_search_into",
    "quantize_rtn8", "quantize_rtn8_into", "matmul_w8", "matmul_w8_into", "select_kernel_w8",
    "gptq_workspace_bytes", "gptq", "gptq_into",
    "select_kernel", "status_string", "version", "MODES", "KERNELS", "SCALE_OPS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libq4.so")

MODES = {"asym": 0, "sym": 1}
KERNELS = {"auto": 0, "gemv": 1, "gemm": 2, "decode": 3}
SCALE_OPS = {"mul": 0, "div": 1}
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
            lib.q4_quantize_rtn_scaled.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, vp, vp]
            lib.q4_quantize_rtn_scaled.restype = ctypes.c_int
            lib.q4_scale_columns.argtypes = [vp, i64, i64, vp, i32, vp, vp]
            lib.q4_scale_columns.restype = ctypes.c_int
            lib.q4_awq_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
            lib.q4_awq_workspace_bytes.restype = ctypes.c_int64
            lib.q4_awq_search.argtypes = [vp, i64, vp, vp, i64, i64, i32, i32, i32, vp, i64, vp, vp, vp,
                                          vp, vp, vp, vp]
            lib.q4_awq_search.restype = ctypes.c_int
            lib.q4_select_kernel.argtypes = [i64, i64, i64, i32]
            lib.q4_select_kernel.restype = ctypes.c_int
            lib.q4_quantize_rtn8.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
            lib.q4_quantize_rtn8.restype = ctypes.c_int
            lib.q4_matmul_w8.argtypes = [vp, i64, i64, i64, i32, i32, vp, vp, vp, vp, i32, vp]
            lib.q4_matmul_w8.restype = ctypes.c_int
            lib.q4_select_kernel_w8.argtypes = [i64, i64, i64, i32]
            lib.q4_select_kernel_w8.restype = ctypes.c_int
            lib.q4_gptq_workspace_bytes.argtypes = [i64, i64, i64, i32]
            lib.q4_gptq_workspace_bytes.restype = ctypes.c_int64
            lib.q4_gptq.argtypes = [vp, i64, vp, i64, i64, i32, i32, ctypes.c_float, vp, i64, vp, vp, vp, vp, vp]
            lib.q4_gptq.restype = ctypes.c_int
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


def select_kernel_w8(M: int, N: int, K: int, g: int) -> str:
    st = library().q4_select_kernel_w8(M, N, K, g)
    if st < 0:
        raise Q4Error(st, "q4_select_kernel_w8")
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


def quantize_rtn_scaled_into(W, s, g: int, mode: str, packed, scales, zeros) -> None:
    """q4_quantize_rtn_scaled (RTN of bf16(W * s)) on caller-provided outputs."""
    import torch
    _check_cuda(W, s, packed, scales, zeros)
    if W.dtype != torch.bfloat16 or W.dim() != 2 or s.dtype != torch.float32 or s.dim() != 1:
        raise ValueError("W must be a 2-D bfloat16 tensor and s a 1-D float32 tensor")
    N, K = W.shape
    if s.shape[0] != K:
        raise ValueError(f"s has {s.shape[0]} entries, W has {K} columns")
    with torch.cuda.device(W.device):
        st = library().q4_quantize_rtn_scaled(_ptr(W), _ptr(s), N, K, g, _mode(mode), _ptr(packed),
                                              _ptr(scales), _ptr(zeros), _stream(W.device))
    if st != 0:
        raise Q4Error(st, "q4_quantize_rtn_scaled")


def quantize_rtn_scaled(W, s, g: int = 128, mode: str = "asym"):
    """RTN quantization of bf16(W * s) -> (packed, scales, zeros)."""
    import torch
    N, K = W.shape
    G = K // g if g > 0 else 0
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=W.device)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=W.device)
    quantize_rtn_scaled_into(W, s, g, mode, packed, scales, zeros)
    return packed, scales, zeros


def scale_columns_into(A, s, op: str, out) -> None:
    """q4_scale_columns: out = bf16(A * s) or bf16(A / s) per column (out may be A)."""
    import torch
    _check_cuda(A, s, out)
    if A.dtype != torch.bfloat16 or out.dtype != torch.bfloat16 or A.dim() != 2 or s.dtype != torch.float32:
        raise ValueError("A and out must be 2-D bfloat16 tensors and s float32")
    if op not in SCALE_OPS:
        raise ValueError(f"op must be one of {sorted(SCALE_OPS)}")
    rows, cols = A.shape
    if tuple(out.shape) != (rows, cols) or s.shape != (cols,):
        raise ValueError("shape mismatch between A, s and out")
    with torch.cuda.device(A.device):
        st = library().q4_scale_columns(_ptr(A), rows, cols, _ptr(s), SCALE_OPS[op], _ptr(out),
                                        _stream(A.device))
    if st != 0:
        raise Q4Error(st, "q4_scale_columns")


def scale_columns(A, s, op: str = "div"):
    import torch
    out = torch.empty_like(A)
    scale_columns_into(A, s, op, out)
    return out


def awq_workspace_bytes(M: int, N: int, K: int, g: int, n_alpha: int = 11) -> int:
    v = int(library().q4_awq_workspace_bytes(M, N, K, g, n_alpha))
    if v < 0:
        raise Q4Error(v, "q4_awq_workspace_bytes")
    return v


def awq_search_into(X, Yref, W, g: int, mode: str, n_alpha: int, workspace, s_out, packed, scales,
                    zeros, errors, best) -> None:
    """q4_awq_search on caller-provided workspace and outputs (no allocation)."""
    import torch
    _check_cuda(X, Yref, W, workspace, s_out, packed, scales, zeros, errors, best)
    if X.dtype != torch.bfloat16 or W.dtype != torch.bfloat16 or Yref.dtype != torch.bfloat16:
        raise ValueError("X, Yref and W must be bfloat16")
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K or tuple(Yref.shape) != (M, N):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}, Yref {tuple(Yref.shape)}")
    if errors.dtype != torch.float64 or best.dtype != torch.int32 or s_out.dtype != torch.float32:
        raise ValueError("errors must be float64, best int32 and s_out float32")
    with torch.cuda.device(W.device):
        st = library().q4_awq_search(_ptr(X), M, _ptr(Yref), _ptr(W), N, K, g, _mode(mode), n_alpha,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _ptr(s_out), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(errors),
                                     _ptr(best), _stream(W.device))
    if st != 0:
        raise Q4Error(st, "q4_awq_search")


def awq_search(X, Yref, W, g: int = 128, mode: str = "asym", n_alpha: int = 11):
    """AWQ-style search on calibration activations X and the layer's unquantized output Yref.

    Returns (s, packed, scales, zeros, errors, best): s the chosen fp32 scales (the weights
    quantized are W * s; divide the activations by s at serve time), errors per grid point
    alpha_i = i / (n_alpha - 1), best the chosen index (device tensors).
    """
    import torch
    M, K = X.shape
    N = W.shape[0]
    G = K // g if g > 0 else 0
    dev = W.device
    ws = torch.empty(awq_workspace_bytes(M, N, K, g, n_alpha), dtype=torch.uint8, device=dev)
    s_out = torch.empty(K, dtype=torch.float32, device=dev)
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, G), dtype=torch.float16, device=dev)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=dev)
    errors = torch.empty(n_alpha, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    awq_search_into(X, Yref, W, g, mode, n_alpha, ws, s_out, packed, scales, zeros, errors, best)
    return s_out, packed, scales, zeros, errors, best


def quantize_rtn8_into(W, g: int, mode: str, codes, scales, zeros) -> None:
    """q4_quantize_rtn8 (8-bit codes, W8A16) on caller-provided outputs (no allocation)."""
    import torch
    _check_cuda(W, codes, scales, zeros)
    if W.dtype != torch.bfloat16 or W.dim() != 2:
        raise ValueError("W must be a 2-D bfloat16 tensor")
    N, K = W.shape
    with torch.cuda.device(W.device):
        st = library().q4_quantize_rtn8(_ptr(W), N, K, g, _mode(mode), _ptr(codes), _ptr(scales),
                                        _ptr(zeros), _stream(W.device))
    if st != 0:
        raise Q4Error(st, "q4_quantize_rtn8")


def quantize_rtn8(W, g: int = 128, mode: str = "sym"):
    """W[N, K] bf16 -> (codes uint8[N, K], scales fp16[N, K/g], zeros uint8[N, K/g])."""
    import torch
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    G = K // g if g > 0 else 0
    codes = torch.empty((N, K), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=W.device)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=W.device)
    quantize_rtn8_into(W, g, mode, codes, scales, zeros)
    return codes, scales, zeros


def matmul_w8_into(X, codes, scales, zeros, g: int, mode: str, Y, kernel: str = "auto") -> None:
    """q4_matmul_w8 on a caller-provided Y (no allocation)."""
    import torch
    _check_cuda(X, codes, scales, zeros, Y)
    if X.dtype != torch.bfloat16 or X.dim() != 2 or Y.dtype != torch.bfloat16:
        raise ValueError("X and Y must be 2-D bfloat16 tensors")
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    M, K = X.shape
    N = codes.shape[0]
    if codes.shape[1] != K or tuple(Y.shape) != (M, N):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, codes {tuple(codes.shape)}, Y {tuple(Y.shape)}")
    with torch.cuda.device(codes.device):
        st = library().q4_matmul_w8(_ptr(X), M, N, K, g, _mode(mode), _ptr(codes), _ptr(scales),
                                    _ptr(zeros), _ptr(Y), KERNELS[kernel], _stream(codes.device))
    if st != 0:
        raise Q4Error(st, "q4_matmul_w8")


def matmul_w8(X, codes, scales, zeros, g: int = 128, mode: str = "sym", kernel: str = "auto"):
    """Y[M, N] = X[M, K] @ dequant(codes, scales, zeros)^T with 8-bit codes, bf16."""
    import torch
    Y = torch.empty((X.shape[0], codes.shape[0]), dtype=torch.bfloat16, device=codes.device)
    matmul_w8_into(X, codes, scales, zeros, g, mode, Y, kernel)
    return Y


def gptq_workspace_bytes(M: int, N: int, K: int, g: int) -> int:
    st = int(library().q4_gptq_workspace_bytes(M, N, K, g))
    if st < 0:
        raise Q4Error(st, "q4_gptq_workspace_bytes")
    return st


def gptq_into(X, W, g: int, mode: str, damp: float, workspace, packed, scales, zeros, info) -> None:
    """q4_gptq on caller-provided workspace and outputs (no allocation)."""
    import torch
    _check_cuda(X, W, workspace, packed, scales, zeros, info)
    if X.dtype != torch.bfloat16 or W.dtype != torch.bfloat16 or X.dim() != 2 or W.dim() != 2:
        raise ValueError("X and W must be 2-D bfloat16 tensors")
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}")
    with torch.cuda.device(W.device):
        st = library().q4_gptq(_ptr(X), M, _ptr(W), N, K, g, _mode(mode), float(damp), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(packed), _ptr(scales),
                               _ptr(zeros), _ptr(info), _stream(W.device))
    if st != 0:
        raise Q4Error(st, "q4_gptq")


def gptq(X, W, g: int = 128, mode: str = "asym", damp: float = 0.01):
    """GPTQ of W[N, K] on calibration rows X[M, K] (bf16) -> (packed, scales, zeros, info)."""
    import torch
    M, K = X.shape
    N = W.shape[0]
    G = K // g if g > 0 else 0
    ws = torch.empty(gptq_workspace_bytes(M, N, K, g), dtype=torch.uint8, device=W.device)
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=W.device)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=W.device)
    info = torch.empty(1, dtype=torch.int32, device=W.device)
    gptq_into(X, W, g, mode, damp, ws, packed, scales, zeros, info)
    return packed, scales, zeros, info
