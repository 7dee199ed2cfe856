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
  16-bit, the matmul in 16-bit.  The oracle computes the product exactly enough to check
  the GPU against: fp64 dequantisation and fp64 accumulation.

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
R9  AWQ-style scaling ("LLM Weight Quantization ...", "GPTQ vs AWQ" toy; "DL S067" §5 "AWQ
    intuition"): a_j = mean over calibration rows of |X[m, j]|; s = a^alpha, divided by
    sqrt(max s * min s); the weights W * s are quantized and 1/s is folded back onto the
    activations; alpha is searched on a grid of [0, 1] by the layer's output error on the
    calibration rows, the first smallest error winning.  In the library's formats:
    a_j is floored at 2^-20 max_j a_j (a channel the calibration never activates gets the
    weakest scale rather than 0; an all-zero X gives s = 1), s is rounded to fp32, the
    quantized weights are bf16(fl32(W[n, j] * s_j)), the activations bf16(fl32(X[m, j] / s_j))
    (IEEE fp32 product / quotient, then round half to even), the grid is i / (n_alpha - 1),
    and the error of alpha is sum (Y_alpha - Y_ref)^2 with Y_alpha the exact product of the
    scaled activations and the dequantised scaled weights and Y_ref the layer's unquantized
    output on the calibration rows (an input, as the calibration activations are).
R10 W8A16 (the INT8 weight-only format of "LLM Weight Quantization ...", "Granularity and
    outliers" and "DL S067" §1's INT8 ranges): the same group-wise RTN with 8-bit codes,
    asymmetric [0, 255] with a uint8 zero-point or symmetric [-127, 127] with zero-point 0,
    fp16 scale, one code per byte (symmetric codes as int8 two's complement); g = K is the
    per-channel case.  [-127, 127] and [-128, 127] give the same symmetric codes, since
    |x| / s <= 127 / (1 - 2^-11) < 127.5.
R11 GPTQ ("LLM Weight Quantization ...", "GPTQ vs AWQ" table and toy; "Model Quantization" §2.1 "GPTQ";
    "DL S067" §4 "GPTQ intuition"): H = X^T X over the calibration rows (the factor 2 of
    "DL S067" cancels in every update), dampened by damp * mean(diag H) on the diagonal with
    damp = 0.01 as in the toy; columns are quantized in order and each column's error,
    divided by the diagonal entry of the current inverse Hessian, is pushed onto the
    remaining columns of its row through that inverse's row, after which the column is
    removed from the inverse.  The toy fixes each row's scale up front from the original
    weights; in the library's group format that reading gives every group the scale and
    zero-point RTN computes from the original weights (so GPTQ changes codes only), and the
    code of a compensated weight w' is clamp(rint(fl32(fl32(w') / scale)) + z): the same fp32
    decision as RTN.  The row updates use the upper Cholesky factor U of H^-1 (U^T U = H^-1),
    whose row i is the current inverse's row i divided by the square root of its diagonal
    entry ("Model Quantization" §2.1: a Cholesky decomposition of the inverse Hessian); the
    toy's route (gptq_toy, closed-form solves on the trailing block of H) gives the same updates.  An all-zero calibration set (mean diag H = 0)
    carries no information: H = I, and GPTQ reduces to RTN.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f32", "quantize_groups", "quantize_rtn_ref", "unpack_codes_ref",
    "dequantize_ref", "round_to_bf16_bits_ref", "dequantize_rounded_ref", "matmul_ref",
    "f32_to_bf16_bits_ref", "awq_alpha_grid", "awq_toy", "channel_absmean_ref", "awq_scale_rule",
    "awq_scales_ref",
    "scale_columns_ref", "quantize_rtn_scaled_ref", "awq_search_ref",
    "quantize8_rtn_ref", "codes8_ref", "dequantize8_ref", "matmul8_ref", "matmul_entries_ref", "tol_ref", "check_matmul",
    "gptq_toy", "gptq_hessian_ref", "gptq_ref", "pack_codes_ref",
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
    packed = pack_codes_ref(q.reshape(N, K))
    return packed, s16.reshape(N, K // g).astype(np.float16), z.reshape(N, K // g).astype(np.uint8)


def pack_codes_ref(q) -> np.ndarray:
    """codes int[N, K] -> packed uint8[N, K/2]: even k in the low nibble, symmetric codes as
    4-bit two's complement (R6)."""
    nib = (np.asarray(q) & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


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


# --------------------------------------------------------------------------- W8A16
Q8_RANGE = {"asym": (0, 255), "sym": (-127, 127)}


def quantize8_rtn_ref(W_bits, g: int = 128, mode: str = "sym"):
    """bf16 W [N, K] -> (codes uint8 [N, K], scales fp16 [N, K/g], zeros uint8 [N, K/g]) (R10):
    the generic group quantizer with 8-bit ranges, fp32 arithmetic, fp16 scales; symmetric
    codes stored as int8 two's complement, zeros 0."""
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    _check_shape(N, K, g)
    x = bf16_bits_to_f32(W_bits).reshape(N, K // g, g)
    q_min, q_max = Q8_RANGE[mode]
    q, s16, z = quantize_groups(x, q_min, q_max, mode)
    codes = (q.reshape(N, K) & 0xFF).astype(np.uint8)
    return codes, s16.astype(np.float16), z.astype(np.uint8)


def codes8_ref(codes, mode: str) -> np.ndarray:
    """uint8 codes -> int64 code values (symmetric: int8 two's complement)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c) if mode == "sym" else c


def dequantize8_ref(codes, scales, zeros, g: int, mode: str) -> np.ndarray:
    """x_hat = fp64(scale) * (q - z), exact in fp64."""
    q = codes8_ref(codes, mode)
    N, K = q.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = np.zeros(s.shape, np.int64) if mode == "sym" else np.asarray(zeros).astype(np.int64)
    if s.shape != (N, K // g) or z.shape != (N, K // g):
        raise ValueError("scales/zeros shape does not match codes and g")
    return (s[..., None] * (q.reshape(N, K // g, g) - z[..., None])).reshape(N, K)


def matmul8_ref(X_bits, codes, scales, zeros, g: int, mode: str):
    """Y_ref = X x_hat^T in fp64 and A = |X| |x_hat|^T (the tolerance scale), as matmul_ref."""
    X = bf16_bits_to_f32(X_bits).astype(np.float64)
    What = dequantize8_ref(codes, scales, zeros, g, mode)
    return X @ What.T, np.abs(X) @ np.abs(What).T


# --------------------------------------------------------------------------- AWQ-style scaling
def awq_alpha_grid(n_alpha: int) -> list:
    """The search grid of R9: alpha_i = i / (n_alpha - 1), i = 0 .. n_alpha - 1 (0 alone when
    n_alpha = 1); 11 points give the toy's grid 0, 0.1, ..., 1."""
    if n_alpha < 1:
        raise ValueError("n_alpha >= 1")
    return [i / (n_alpha - 1) if n_alpha > 1 else 0.0 for i in range(n_alpha)]


def awq_toy(W, X, qdq, n_alpha: int = 11):
    """Activation-aware scaling of the pages' toy (R9) in fp64, for any quantizer.

    W [rows, d] weights, X [m, d] calibration activations, qdq(Ws) -> the quantized then
    dequantized Ws.  Every alpha of the grid is scored: the channel scales come from the same
    rule as the library-format search (awq_scale_rule on the mean |x| of each channel), the
    candidate weights are qdq(W s) with 1/s folded back onto them, and the score is the
    calibration output error ||X W^T - X Q^T||.  The first alpha with the smallest score wins.
    Returns (Q of the winner, its alpha, the scores).
    """
    W = np.asarray(W, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    grid = awq_alpha_grid(n_alpha)
    a = np.abs(X).mean(axis=0)
    cands = [qdq(W * s) / s for s in (awq_scale_rule(a, al) for al in grid)]
    scores = np.array([np.linalg.norm(X @ (W - Q).T) for Q in cands])
    k = int(np.argmin(scores))                                 # first smallest
    return cands[k], grid[k], scores


def f32_to_bf16_bits_ref(x32) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round half to even on the bit pattern (R3): add half of the
    dropped range, plus one when the kept part is odd, and keep the top 16 bits.  Exact for
    every finite fp32 value, subnormals included; a result beyond bf16's range is +-inf."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    if not np.all(np.isfinite(np.asarray(x32, dtype=np.float32))):
        raise ValueError("NaN or Inf input is outside the method's domain")
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def channel_absmean_ref(X_bits) -> np.ndarray:
    """a_j = mean over rows m of |X[m, j]| (R9), fp64."""
    X = bf16_bits_to_f32(X_bits).astype(np.float64)
    return np.abs(X).mean(axis=0)


AWQ_FLOOR = 2.0 ** -20


def awq_scale_rule(a, alpha: float) -> np.ndarray:
    """fp64 channel scales of R9: a floored at 2^-20 max(a), raised to alpha and divided by the
    geometric mean of the largest and smallest, sqrt(max(a^alpha) min(a^alpha)), so the scales
    sit around 1 ("DL S067" §5 "AWQ intuition": weight columns of salient channels scaled up,
    activations down).  An all-zero a gives 1 everywhere."""
    a = np.asarray(a, dtype=np.float64)
    amax = a.max()
    if amax == 0.0:
        return np.ones(a.shape, np.float64)
    p = np.maximum(a, AWQ_FLOOR * amax) ** alpha
    return p / np.sqrt(p.max() * p.min())


def awq_scales_ref(a, alpha: float) -> np.ndarray:
    """The library's channel scales: awq_scale_rule rounded to fp32 (R9)."""
    return awq_scale_rule(a, alpha).astype(np.float32)


def scale_columns_ref(A_bits, s32, op: str) -> np.ndarray:
    """bf16(fl32(A[r, j] * s_j)) for op="mul", bf16(fl32(A[r, j] / s_j)) for op="div" (R9):
    one IEEE fp32 product or quotient (numpy float32), then round half to even to bf16."""
    A = bf16_bits_to_f32(A_bits)
    s = np.asarray(s32, dtype=np.float32)
    if op == "mul":
        v = A * s[None, :]
    elif op == "div":
        v = A / s[None, :]
    else:
        raise ValueError(f"unknown op {op!r}")
    return f32_to_bf16_bits_ref(v)


def quantize_rtn_scaled_ref(W_bits, s32, g: int = 128, mode: str = "asym"):
    """RTN quantization of bf16(fl32(W * s)) (R9): the weights of AWQ-style scaling."""
    return quantize_rtn_ref(scale_columns_ref(W_bits, s32, "mul"), g, mode)


def awq_search_ref(W_bits, X_bits, Yref_bits, g: int = 128, mode: str = "asym", n_alpha: int = 11):
    """AWQ-style scaling in the library's formats (R9).

    W_bits [N, K] weights, X_bits [M, K] calibration activations, Yref_bits [M, N] the layer's
    unquantized output on them (bf16 bit patterns).  For alpha_i = i / (n_alpha - 1): scales
    s_i (awq_scales_ref), quantize bf16(W * s_i), scale the activations bf16(X / s_i), and
    error_i = sum (Y_i - Y_ref)^2 with Y_i their exact product.  Returns a dict with the best
    index (first smallest error), alphas, errors, the scales of every alpha (fp32) and the
    best alpha's packed / scales / zeros.
    """
    a = channel_absmean_ref(X_bits)
    Yref = bf16_bits_to_f32(Yref_bits).astype(np.float64)
    alphas = awq_alpha_grid(n_alpha)
    errs, svals, quants = [], [], []
    for al in alphas:
        s = awq_scales_ref(a, al)
        q = quantize_rtn_scaled_ref(W_bits, s, g, mode)
        Xs = scale_columns_ref(X_bits, s, "div")
        Y, _ = matmul_ref(Xs, *q, g, mode)
        errs.append(float(((Y - Yref) ** 2).sum()))
        svals.append(s)
        quants.append(q)
    best = int(np.argmin(errs))             # first smallest
    return {"best": best, "alphas": alphas, "errors": np.array(errs), "scales": np.array(svals),
            "quant": quants[best], "absmean": a}


# --------------------------------------------------------------------------- GPTQ
def gptq_toy(W, X, quant_col, damp=0.01):
    """GPTQ of the pages' toy (R11) in fp64, for any column quantizer.

    W [rows, d] weights, X [m, d] calibration activations, quant_col(i, v) -> the quantized then
    dequantized values v of column i (one per row, scales fixed up front by the caller).
    H = X^T X with damp * mean(diag H) added to its diagonal.  Columns are fixed in order.
    Once column i is fixed with rounding error e = w_i - q_i, the columns F = i+1 .. d-1 not
    yet fixed move by the minimiser of the calibration output error ||X delta||^2 =
    delta^T H delta under delta_i = -e ("DL S067" §4 "GPTQ intuition"): setting the gradient
    in delta_F to zero gives H_FF delta_F = e H_Fi, so w_F += e * solve(H_FF, H_Fi).  By the
    block-inverse identity this is the pages' update through the inverse Hessian of the
    columns i.. (its row i divided by its diagonal entry equals -H_iF H_FF^-1).  The solve
    vectors depend only on H, so every row moves at once.  Returns Q [rows, d].
    """
    w = np.array(W, dtype=np.float64)                # compensated in place
    X = np.asarray(X, dtype=np.float64)
    H = X.T @ X
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    d = w.shape[1]
    Q = np.empty_like(w)
    for i in range(d):
        Q[:, i] = quant_col(i, w[:, i])
        if i + 1 < d:
            v = np.linalg.solve(H[i + 1:, i + 1:], H[i + 1:, i])
            w[:, i + 1:] += np.outer(w[:, i] - Q[:, i], v)
    return Q


def gptq_hessian_ref(X_bits, damp: float = 0.01) -> np.ndarray:
    """H = X^T X (fp64, X the bf16 calibration rows) + damp * mean(diag H) * I; I when X is all
    zero (R11)."""
    X = bf16_bits_to_f32(X_bits).astype(np.float64)
    H = X.T @ X
    m = np.mean(np.diag(H))
    if m == 0.0:
        return np.eye(H.shape[0])
    return H + damp * m * np.eye(H.shape[0])


def gptq_ref(W_bits, X_bits, g: int = 128, mode: str = "asym", damp: float = 0.01,
             return_quotients: bool = False):
    """GPTQ of a bf16 weight W[N, K] on bf16 calibration rows X[M, K], in the library's INT4
    group format (R11): (packed uint8[N, K/2], scales fp16[N, K/g], zeros uint8[N, K/g]).

    The scales and zero-points are RTN's on the original weights (fixed up front).  The sweep
    runs in fp64 over all rows at once, column by column, with U the upper Cholesky factor of
    H^-1: code of the compensated column (fp32 decision, as RTN), err = (w_i - x_hat_i) / U_ii,
    w[:, i+1:] -= err U[i, i+1:].  With return_quotients the fp32 quotients fl32(w') / scale the
    codes were rounded from are returned as a fourth value (float32 [N, K]).
    """
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    _check_shape(N, K, g)
    if np.asarray(X_bits).shape[1:] != (K,):
        raise ValueError("X must have K columns")
    q_min, q_max = {"asym": (0, 15), "sym": (-8, 7)}[mode]
    W32 = bf16_bits_to_f32(W_bits)
    _, s16, z = quantize_groups(W32.reshape(N, K // g, g), q_min, q_max, mode)
    s32 = s16.astype(np.float32)                              # [N, G]
    s64 = s32.astype(np.float64)
    H = gptq_hessian_ref(X_bits, damp)
    U = np.linalg.cholesky(np.linalg.inv(H)).T               # upper, U^T U = H^-1
    w = W32.astype(np.float64)
    q = np.empty((N, K), dtype=np.int64)
    quots = np.empty((N, K), dtype=np.float32) if return_quotients else None
    for i in range(K):
        G = i // g
        quot = w[:, i].astype(np.float32) / s32[:, G]         # fl32(fl32(w') / scale)
        if return_quotients:
            quots[:, i] = quot
        r = np.clip(np.rint(quot), np.float32(-2.0 ** 40), np.float32(2.0 ** 40)).astype(np.int64)
        q[:, i] = np.clip(r + z[:, G], q_min, q_max)
        what = s64[:, G] * (q[:, i] - z[:, G])
        err = (w[:, i] - what) / U[i, i]
        w[:, i + 1:] -= np.outer(err, U[i, i + 1:])
    if return_quotients:
        return pack_codes_ref(q), s16.astype(np.float16), z.astype(np.uint8), quots
    return pack_codes_ref(q), s16.astype(np.float16), z.astype(np.uint8)


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
