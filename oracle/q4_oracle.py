"""CPU oracle for group-wise affine INT4 round-to-nearest quantization and the W4A16 matmul.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library's product path
(the HIP kernels behind the C ABI) never calls, links or imports it, and this module
shares no code, table or helper with that path.

Plain numpy, written to be checked by eye against the pages:

* affine (asymmetric) quantization -- "DL S067 · Quantization — INT8, INT4, GPTQ, AWQ",
  §1 "The core math": scale = (beta - alpha) / (q_max - q_min),
  z = round(q_min - alpha / scale), q = clip(round(x / scale) + z, q_min, q_max),
  x_hat = scale * (q - z); the same formulas appear in "Model Quantization" §1
  (Affine Quantization) and in the vocabulary of "LLM Weight Quantization - GPTQ, AWQ,
  SmoothQuant, FP8 & INT4/INT8 Trade-offs" ("Scale and zero-point");
* symmetric quantization -- same section of "DL S067": drop the zero-point and use
  scale = max|x| / q_max;
* group-wise granularity -- "Model Quantization" §1 (Group-wise Quantization) and
  "DL S067" §2 "Per-tensor vs per-channel vs per-group": one scale (and zero) per group of
  g consecutive weights along the input dimension of each output row, g = 128 by default;
* W4A16 -- "LLM Weight Quantization ...", "The vocabulary": 4-bit weights dequantised to
  16-bit, the matmul in 16-bit.  The oracle computes the product exactly enough to judge
  the GPU: fp64 dequantisation and fp64 accumulation.

Readings of points the pages leave open (each one is listed with its reason in the
design notes of the repository):

R1  alpha = min(group) and beta = max(group), both extended to include 0, so the zero
    point lies in [q_min, q_max] and 0 is exactly representable.
R2  asymmetric INT4 uses [q_min, q_max] = [0, 15] and scale = (beta - alpha) / 15;
    symmetric INT4 uses [-8, 7] and scale = max|x| / 7 (q_max = 7).
R3  "round" is round-half-to-even (numpy/torch round, which the pages' snippets use);
    conversions fp32 -> fp16 and -> bf16 also round to nearest even.
R4  arithmetic: the weight is widened to fp32 (exact for bf16), the scale is computed in
    IEEE fp32, stored as fp16 (saturated at 65504; an fp16 scale of 0 becomes 1.0), and the
    codes use the fp32 quotient x / scale_fp16 rounded half-to-even.
R5  z = clamp(rint(0 - fl32(alpha / scale)), q_min, q_max); symmetric mode stores z = 0.
R6  codes are stored two per byte, even k in the low nibble; symmetric codes are stored as
    4-bit two's complement.
R7  x_hat = fp64(scale_fp16) * (q - z)  (exact in fp64).
R8  the standalone dequantisation returns x_hat rounded once to bf16 or fp16, round half
    to even (R3); an fp16 result beyond the fp16 range becomes +-inf as IEEE rounding
    says.  x_hat has at most 15 significant bits and lies in bf16's normal range (or is 0).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f32", "quantize_groups", "quantize_rtn_ref", "unpack_codes_ref",
    "dequantize_ref", "round_to_bf16_bits_ref", "dequantize_rounded_ref", "matmul_ref", "matmul_entries_ref", "tol_ref", "check_matmul",
    "bits_per_weight", "weight_bytes", "format_math_row",
]

F16_MAX = np.float32(65504.0)


# --------------------------------------------------------------------------- formats
def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32.  Exact: bf16 is the top half of fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _to_f16_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 with round-half-to-even (numpy's float32 -> float16 conversion)."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------- generic core
def quantize_groups(xg, q_min: int, q_max: int, mode: str, scale_format: str = "fp16",
                    dtype=np.float32):
    """Round-to-nearest quantization of every group along the last axis of ``xg``.

    Follows "DL S067 · Quantization", §1 "The core math" (asymmetric and symmetric
    formulas), with readings R1-R5 above.

    xg            array (..., g): each slice along the last axis is one group.
    q_min, q_max  integer code range, e.g. (0, 15) asymmetric INT4, (-8, 7) symmetric INT4,
                  (-127, 127) the INT8 symmetric range of the worked example.
    mode          "asym" (scale and zero-point) or "sym" (zero-point dropped).
    scale_format  "fp16": the scale is stored as fp16 (R4); "exact": the scale stays in
                  ``dtype`` (used to reproduce the pages' fp64 snippets).
    dtype         arithmetic precision, np.float32 (the library's) or np.float64.

    Returns (q int64 (..., g), scale (..., ) in fp16 or dtype, z int64 (..., )).
    """
    dt = np.dtype(dtype).type
    x = np.asarray(xg, dtype=dt)
    if not np.all(np.isfinite(x)):
        raise ValueError("NaN or Inf input is outside the method's domain")
    if mode == "asym":
        alpha = np.minimum(x.min(axis=-1), dt(0))            # R1
        beta = np.maximum(x.max(axis=-1), dt(0))
        scale = (beta - alpha) / dt(q_max - q_min)           # §1: (beta-alpha)/(qmax-qmin)
    elif mode == "sym":
        alpha = None
        scale = np.abs(x).max(axis=-1) / dt(q_max)           # §1 symmetric: max|x| / q_max
    else:
        raise ValueError(f"unknown mode {mode!r}")

    if scale_format == "fp16":
        s16 = _to_f16_rne(np.minimum(scale.astype(np.float32), F16_MAX))   # R4
        s16 = np.where(s16 == np.float16(0), np.float16(1.0), s16)
        stored = s16
        s = s16.astype(dt)
    elif scale_format == "exact":
        s = np.where(scale == dt(0), dt(1), scale)
        stored = s
    else:
        raise ValueError(f"unknown scale_format {scale_format!r}")

    if mode == "asym":
        ratio = alpha / s                                     # fl(alpha / scale)
        z = np.clip(np.rint(dt(q_min) - ratio), q_min, q_max).astype(np.int64)   # R5
    else:
        z = np.zeros(s.shape, dtype=np.int64)

    quot = x / s[..., None]                                   # fl(x / scale)
    # rint(quot) is limited to +-2^40 before the integer conversion only so that a huge
    # quotient (saturated scale) cannot overflow int64; the clip below gives the same code.
    r = np.clip(np.rint(quot), dt(-2.0 ** 40), dt(2.0 ** 40)).astype(np.int64)
    q = np.clip(r + z[..., None], q_min, q_max)
    return q, stored, z


# --------------------------------------------------------------------------- INT4 API
def _check_shape(N: int, K: int, g: int):
    if N < 1 or K < 1 or K % 2 or g < 1 or K % g:
        raise ValueError(f"bad shape N={N} K={K} g={g}")


def quantize_rtn_ref(W_bits, g: int = 128, mode: str = "asym"):
    """INT4 group-wise RTN of a bf16 weight W[N, K] (bit patterns).

    Returns (packed uint8[N, K/2], scales fp16[N, K/g], zeros uint8[N, K/g]); see R1-R6.
    Groups are g consecutive weights along K within one row ("DL S067" §2 group view
    (out, G, gs); scale shape (out, G)).
    """
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    _check_shape(N, K, g)
    x = bf16_bits_to_f32(W_bits).reshape(N, K // g, g)
    if mode == "asym":
        q, s16, z = quantize_groups(x, 0, 15, "asym")
    elif mode == "sym":
        q, s16, z = quantize_groups(x, -8, 7, "sym")
    else:
        raise ValueError(f"unknown mode {mode!r}")
    nib = (q.reshape(N, K) & 0xF).astype(np.uint8)            # R6: two's complement nibble
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, s16.reshape(N, K // g).astype(np.float16), z.reshape(N, K // g).astype(np.uint8)


def unpack_codes_ref(packed, mode: str) -> np.ndarray:
    """packed uint8[N, K/2] -> codes int64[N, K]; even k from the low nibble (R6)."""
    p = np.asarray(packed, dtype=np.uint8)
    N, H = p.shape
    codes = np.empty((N, 2 * H), dtype=np.int64)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    if mode == "sym":
        codes = np.where(codes >= 8, codes - 16, codes)        # 4-bit two's complement
    return codes


def dequantize_ref(packed, scales, zeros, g: int, mode: str) -> np.ndarray:
    """x_hat[n, k] = fp64(scale[n, k/g]) * (q[n, k] - z[n, k/g])   (R7, exact in fp64)."""
    q = unpack_codes_ref(packed, mode)
    N, K = q.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = np.zeros(s.shape, np.int64) if mode == "sym" else np.asarray(zeros).astype(np.int64)
    if s.shape != (N, K // g) or z.shape != (N, K // g):
        raise ValueError("scales/zeros shape does not match packed and g")
    qg = q.reshape(N, K // g, g)
    return (s[..., None] * (qg - z[..., None])).reshape(N, K)


BF16_MIN_NORMAL = 2.0 ** -126
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16_bits_ref(x) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), rounding the exact value half to even (R3).

    bf16 keeps 8 significant bits: write x = m * 2**e with 0.5 <= |m| < 1, round m * 2**8 to
    an integer (ties to even) and scale back.  Defined for 0 and for results in bf16's
    normal range, which covers every dequantised weight (R8); anything else raises.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    a = np.abs(r)
    if not np.all((a == 0) | ((a >= BF16_MIN_NORMAL) & (a <= BF16_MAX))):
        raise ValueError("value outside the range this rounding is defined for")
    # r has at most 8 significant bits and a normal exponent: exact in fp32, and its bf16
    # pattern is the top half of the fp32 pattern.
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def dequantize_rounded_ref(packed, scales, zeros, g: int, mode: str, out: str = "bf16"):
    """x_hat (R7) rounded once to the output format (R8): bf16 bit patterns (uint16) for
    out="bf16", a float16 array for out="f16"."""
    xhat = dequantize_ref(packed, scales, zeros, g, mode)
    if out == "bf16":
        return round_to_bf16_bits_ref(xhat)
    if out == "f16":
        with np.errstate(over="ignore"):
            return xhat.astype(np.float16)       # numpy rounds fp64 -> fp16 half to even
    raise ValueError(f"unknown output format {out!r}")


def matmul_ref(X_bits, packed, scales, zeros, g: int, mode: str):
    """Y_ref[m, n] = sum_k X[m, k] * x_hat[n, k] in fp64, and A[m, n] = sum_k |X[m, k] x_hat[n, k]|.

    A is the scale of the tolerance: tol = 8e-3 * A + 1e-6 per element.
    """
    X = bf16_bits_to_f32(X_bits).astype(np.float64)
    What = dequantize_ref(packed, scales, zeros, g, mode)
    Y = X @ What.T
    A = np.abs(X) @ np.abs(What).T
    return Y, A


def matmul_entries_ref(X_bits, packed, scales, zeros, g: int, mode: str, m_idx, n_idx):
    """Y_ref and A at sampled (m, n) positions only, one dot product each (for full-size runs)."""
    m_idx = np.asarray(m_idx, dtype=np.int64)
    n_idx = np.asarray(n_idx, dtype=np.int64)
    rows = np.unique(n_idx)
    sub = dequantize_ref(np.asarray(packed)[rows], np.asarray(scales)[rows],
                         None if mode == "sym" else np.asarray(zeros)[rows], g, mode)
    pos = {int(r): i for i, r in enumerate(rows)}
    X = bf16_bits_to_f32(np.asarray(X_bits)[np.unique(m_idx)]).astype(np.float64)
    mpos = {int(r): i for i, r in enumerate(np.unique(m_idx))}
    Y = np.empty(len(m_idx)); A = np.empty(len(m_idx))
    for t, (m, n) in enumerate(zip(m_idx, n_idx)):
        x = X[mpos[int(m)]]
        w = sub[pos[int(n)]]
        Y[t] = np.dot(x, w)
        A[t] = np.dot(np.abs(x), np.abs(w))
    return Y, A


def tol_ref(A) -> np.ndarray:
    """Per-element acceptance bound |Y - Y_ref| <= 8e-3 * A + 1e-6."""
    return 8e-3 * np.asarray(A, dtype=np.float64) + 1e-6


def check_matmul(Y_gpu_f64, Y_ref, A):
    """Return (ok, max tolerance usage = max |Y - Y_ref| / tol)."""
    err = np.abs(np.asarray(Y_gpu_f64, dtype=np.float64) - Y_ref)
    usage = err / tol_ref(A)
    worst = float(usage.max()) if usage.size else 0.0
    return bool(np.all(usage <= 1.0)), worst


# --------------------------------------------------------------------------- format math
def bits_per_weight(g: int, mode: str, scale_bits: int = 16, zero_bits: int = 8) -> float:
    """Storage per weight: 4 code bits + per-group scale (+ zero-point in asymmetric mode).

    "DL S067" §2 counts 4 + 16/128 = 4.125 for an fp16 scale alone; this format adds an
    8-bit zero per group in asymmetric mode.
    """
    extra = scale_bits + (zero_bits if mode == "asym" else 0)
    return 4.0 + extra / g


def weight_bytes(N: int, K: int, g: int, mode: str) -> int:
    """Exact bytes of packed codes + fp16 scales (+ uint8 zeros) for W[N, K]."""
    G = K // g
    return N * K // 2 + 2 * N * G + (N * G if mode == "asym" else 0)


def format_math_row(params: float, bits_per_w: float, hbm_bytes: float = 80e9,
                    bandwidth: float = 3.35e12, usable: float = 0.9):
    """Weights-only decode ceiling ("LLM Weight Quantization ...", format-math snippet).

    bytes = params * bits / 8; minimum GPUs = ceil(bytes / (HBM * usable));
    tokens/s at batch 1 <= bandwidth * gpus / bytes; at 8 GPUs = bandwidth * 8 / bytes.
    Returns (GB, gpus, ceiling at min GPUs, ceiling at 8 GPUs or None).
    """
    nbytes = params * bits_per_w / 8
    gpus = int(np.ceil(nbytes / (hbm_bytes * usable)))
    ceiling = bandwidth * gpus / nbytes
    at8 = bandwidth * 8 / nbytes if gpus <= 8 else None
    return nbytes / 1e9, gpus, ceiling, at8
