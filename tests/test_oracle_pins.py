"""Pins of the CPU oracle against what the pages print (worked example, printed tables,
format math) and against hand-worked examples of the pages' formulas.

Each fixture under tests/golden/ carries its citation.  None of these values comes from
the HIP library.
"""
import json
import os

import numpy as np
import pytest

from oracle import q4_oracle as orc
from synth import f64_to_bf16_bits


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- worked example (INT8 sym)
def test_worked_example_exact_scale(golden_dir):
    gx = _load(golden_dir, "worked_example_int8_sym.json")
    x = np.array([gx["x"]], dtype=np.float64)
    lo, hi = gx["q_range"]
    q, s, z = orc.quantize_groups(x, lo, hi, "sym", "exact", np.float64)
    assert q[0].tolist() == gx["codes"]
    assert int(z[0]) == 0
    assert round(float(s[0]), 5) == gx["scale_printed"]
    xhat = q[0] * s[0]
    assert np.round(xhat, gx["xhat_decimals"]).tolist() == gx["xhat_printed"]
    err = np.abs(x[0] - xhat).max()
    assert round(err, gx["err_decimals"]) == gx["err_inf_printed"]
    assert np.all(np.abs(x[0] - xhat) <= s[0] / 2)


def test_worked_example_fp16_scale(golden_dir):
    gx = _load(golden_dir, "worked_example_int8_sym.json")
    x = np.array([gx["x"]], dtype=np.float32)
    lo, hi = gx["q_range"]
    q, s16, z = orc.quantize_groups(x, lo, hi, "sym", "fp16", np.float32)
    assert q[0].tolist() == gx["codes"]
    assert int(s16.view(np.uint16)[0]) == 0x20D6
    sf = float(s16[0])
    xhat = q[0].astype(np.float64) * sf
    err = np.abs(x[0].astype(np.float64) - xhat)
    assert np.all(err <= sf / 2)
    assert round(err.max(), gx["err_decimals"]) == gx["err_inf_printed"]


# ----------------------------------------------------------------- page-3 printed table
def _granularity_tensors():
    """Synthetic tensors of the 'Granularity and outliers' snippet, drawn in its order."""
    rng = np.random.default_rng(0)
    W = rng.normal(0, 0.02, (1024, 1024))
    W[:8] *= 6
    X = rng.normal(0, 1, (256, 1024))
    ch = rng.choice(1024, 6, replace=False)
    X[:, ch] *= 50
    return W, X


def _qdq_sym(x, bits, group_shape, scale_format="exact", dtype=np.float64):
    qmax = 2 ** (bits - 1) - 1
    q, s, _ = orc.quantize_groups(x.reshape(group_shape), -qmax - 1, qmax, "sym", scale_format, dtype)
    return (q * np.asarray(s, dtype=np.float64)[..., None]).reshape(x.shape)


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(a)


def test_granularity_table(golden_dir):
    gt = _load(golden_dir, "granularity_table.json")
    W, X = _granularity_tensors()
    d = gt["decimals"]
    we = gt["weight_error"]
    assert round(_rel(W, _qdq_sym(W, 8, (1, 1, -1))), d) == we["int8_per_tensor"]
    assert round(_rel(W, _qdq_sym(W, 8, (1024, 1, 1024))), d) == we["int8_per_channel"]
    assert round(_rel(W, _qdq_sym(W, 4, (1024, 1, 1024))), d) == we["int4_per_channel"]
    assert round(_rel(W, _qdq_sym(W, 4, (1024, 8, 128))), d) == we["int4_group128"]
    Y = X @ W.T
    Yq = X @ _qdq_sym(W, 8, (1024, 1, 1024)).T
    assert round(_rel(Y, Yq), d) == gt["output_error"]["weight_only_w8a16"]


def test_granularity_int4_g128_with_fp16_scale(golden_dir):
    """Storing the group scale as fp16 (fp32 arithmetic) leaves the printed g=128 error unchanged."""
    gt = _load(golden_dir, "granularity_table.json")
    W, _ = _granularity_tensors()
    W32 = W.astype(np.float32)
    err = _rel(W, _qdq_sym(W32, 4, (1024, 8, 128), "fp16", np.float32))
    assert round(err, gt["decimals"]) == gt["weight_error"]["int4_group128"]


def test_toy_rtn_3bit(golden_dir):
    gt = _load(golden_dir, "toy_rtn_3bit.json")
    rng = np.random.default_rng(1)
    d, rows, n = 128, 64, 1024
    mix = rng.normal(0, 1, (d, d)) / np.sqrt(d)
    factors = np.ones(d)
    factors[rng.choice(d, 4, replace=False)] = 8.0

    def acts(m):
        a = rng.normal(0, 1, (m, d)) @ mix
        b = 0.3 * rng.normal(0, 1, (m, d))
        return (a + b) * factors

    _xcal = acts(n)
    xtest = acts(n)
    W = rng.normal(0, 0.05, (rows, d))
    Q = _qdq_sym(W, 3, (rows, 1, d))
    out_err = np.linalg.norm(xtest @ W.T - xtest @ Q.T) / np.linalg.norm(xtest @ W.T)
    assert round(out_err, gt["rtn_output_decimals"]) == gt["rtn_output_error"]
    assert round(_rel(W, Q), gt["rtn_weight_decimals"]) == gt["rtn_weight_error"]


# ----------------------------------------------------------------- format math
def test_format_math_table(golden_dir):
    gt = _load(golden_dir, "format_math.json")
    for fmt, model, bits, params, gb, gpus, ceil_min, ceil8 in gt["rows"]:
        got_gb, got_gpus, got_ceil, got_at8 = orc.format_math_row(params, bits)
        assert round(got_gb) == gb, (fmt, model)
        assert got_gpus == gpus, (fmt, model)
        assert round(got_ceil) == ceil_min, (fmt, model)
        if ceil8 is None:
            assert got_at8 is None
        else:
            assert round(got_at8) == ceil8, (fmt, model)


def test_bits_per_weight_closed_form():
    # "DL S067" §2: 4 + 16/128 = 4.125 bits for an fp16 scale per 128 weights.
    assert orc.bits_per_weight(128, "sym") == 4.125
    assert orc.bits_per_weight(128, "asym") == 4.0 + 24 / 128
    assert orc.weight_bytes(28672, 8192, 128, "asym") == 117440512 + 3670016 + 1835008
    # bytes / (params * bits / 8) is exactly 1 for every shape
    for N, K, g, mode in [(11008, 4096, 128, "asym"), (4096, 4096, 128, "sym"), (8192, 8192, 32, "asym")]:
        assert orc.weight_bytes(N, K, g, mode) * 8 == N * K * orc.bits_per_weight(g, mode)


# ----------------------------------------------------------------- hand-worked INT4 examples
@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_hand_example(golden_dir, mode):
    ex = _load(golden_dir, "hand_examples.json")[mode]
    W_bits = f64_to_bf16_bits(np.array([ex["x"]]))
    assert np.array_equal(orc.bf16_bits_to_f32(W_bits).astype(np.float64), np.array([ex["x"]]))
    packed, scales, zeros = orc.quantize_rtn_ref(W_bits, g=8, mode=mode)
    assert float(scales[0, 0]) == ex["scale"]
    assert int(zeros[0, 0]) == ex["zero"]
    assert [f"0x{b:02X}" for b in packed[0]] == ex["packed_hex"]
    assert orc.unpack_codes_ref(packed, mode)[0].tolist() == ex["codes"]
    xhat = orc.dequantize_ref(packed, scales, zeros, 8, mode)
    assert xhat[0].tolist() == ex["xhat"]


# ----------------------------------------------------------------- layout pins
def test_nibble_order_and_sign():
    # scale (15-0)/15 = 1, zero 0: codes (1, 2) at k = 0, 1 -> byte 0x21 (even k in the low nibble)
    W_bits = f64_to_bf16_bits(np.array([[1.0, 2.0] + [0.0] * 29 + [15.0]]))
    p, s, z = orc.quantize_rtn_ref(W_bits, g=32, mode="asym")
    assert float(s[0, 0]) == 1.0 and int(z[0, 0]) == 0
    assert p[0, 0] == 0x21 and p[0, 15] == 0xF0
    # symmetric: max|x| = 7 -> scale 1; code -1 -> nibble 0xF, code 7 -> 0x7
    W_bits = f64_to_bf16_bits(np.array([[-1.0, 7.0] + [0.0] * 30]))
    p, s, z = orc.quantize_rtn_ref(W_bits, g=32, mode="sym")
    assert float(s[0, 0]) == 1.0 and int(z[0, 0]) == 0 and p[0, 0] == 0x7F


def test_one_hot_reads_back_single_weights():
    rng = np.random.default_rng(5)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (6, 64)))
    for mode in ("asym", "sym"):
        packed, scales, zeros = orc.quantize_rtn_ref(W_bits, g=32, mode=mode)
        codes = orc.unpack_codes_ref(packed, mode)
        X_bits = f64_to_bf16_bits(np.eye(64))
        Y, A = orc.matmul_ref(X_bits, packed, scales, zeros, 32, mode)
        for n in range(6):
            for k in range(64):
                zz = 0 if mode == "sym" else int(zeros[n, k // 32])
                assert Y[k, n] == float(scales[n, k // 32]) * (codes[n, k] - zz)
                assert A[k, n] == abs(Y[k, n])


# --------------------------------------------------------------------------- rounded dequantisation
BF16_HAND_CASES = {
        1.0 + 2.0 ** -8: 0x3F80,                  # half an ulp above 1: tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,              # 1.5 ulp: tie -> 1 + 2^-6 (even)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,     # just above the tie -> up
        -(1.0 + 2.0 ** -8): 0xBF80,
        0.0: 0x0000,
        255.5: 0x4380,                            # 255.5 -> 256 (9 significant bits needed)
        3.0 * 2.0 ** -24: 0x3440,                 # smallest fp16 scale times 3: exact
        65504.0 * 15: 0x4970,                     # largest |x_hat|: 982560 -> 983040
}


def _torch_bf16_cases():
    import torch
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(100000) * np.exp2(rng.uniform(-100, 100, 100000))).astype(np.float32)
    ties = (rng.integers(1, 2 ** 16, 20000) * 2 + 1).astype(np.float64) * 2.0 ** -9   # odd/2^9: many ties
    x = np.concatenate([x, ties.astype(np.float32)])
    return x, torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rounding_pins_hold(o) -> bool:
    """The bf16 rounding pins below in compact form (used by the mutation tests)."""
    got = o.round_to_bf16_bits_ref(np.array(list(BF16_HAND_CASES)))
    if [int(v) for v in got] != list(BF16_HAND_CASES.values()):
        return False
    x, want = _torch_bf16_cases()
    return bool(np.array_equal(o.round_to_bf16_bits_ref(x.astype(np.float64)), want))


def test_bf16_rounding_hand_values():
    """bf16 keeps 8 significant bits; ties go to the even neighbour (ulp at 1 is 2^-7)."""
    got = orc.round_to_bf16_bits_ref(np.array(list(BF16_HAND_CASES)))
    assert [int(v) for v in got] == list(BF16_HAND_CASES.values())


def test_bf16_rounding_matches_torch_conversion():
    """Against an independent routine: torch's fp32 -> bf16 conversion (round to nearest
    even) on values exact in fp32 across bf16's normal exponent range."""
    x, want = _torch_bf16_cases()
    assert np.array_equal(orc.round_to_bf16_bits_ref(x.astype(np.float64)), want)


def test_bf16_rounding_rejects_out_of_range():
    for v in (2.0 ** -130, 1e39, np.inf, np.nan):
        with pytest.raises(ValueError):
            orc.round_to_bf16_bits_ref(np.array([v]))


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_dequantize_rounded_exact_when_representable(mode):
    """Power-of-two scales make every x_hat = 2^e (q - z) exact in bf16 and fp16 (|q - z| <= 15
    needs 4 significant bits), so the rounded output must equal x_hat itself."""
    rng = np.random.default_rng(5)
    N, K, g = 6, 256, 64
    q = rng.integers(0, 16, (N, K))
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    scales = np.exp2(rng.integers(-20, 10, (N, K // g))).astype(np.float16)
    zeros = rng.integers(0, 16, (N, K // g)).astype(np.uint8)
    codes = q if mode == "asym" else np.where(q >= 8, q - 16, q)
    z = zeros.astype(np.int64) if mode == "asym" else np.zeros_like(zeros, dtype=np.int64)
    xhat = scales.astype(np.float64).repeat(g, axis=1) * (codes - z.repeat(g, axis=1))
    b = orc.dequantize_rounded_ref(packed, scales, zeros, g, mode, "bf16")
    assert np.array_equal(orc.bf16_bits_to_f32(b).astype(np.float64), xhat)
    h = orc.dequantize_rounded_ref(packed, scales, zeros, g, mode, "f16")
    assert h.dtype == np.float16 and np.array_equal(h.astype(np.float64), xhat)


def test_dequantize_rounded_f16_matches_torch_and_overflows():
    """fp16 output against torch's conversion of the (fp32-exact) products; products beyond
    65504 (plus half an ulp) become inf."""
    import torch
    rng = np.random.default_rng(9)
    N, K, g = 4, 128, 32
    packed = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    scales = np.array(rng.uniform(0.5, 30000, (N, K // g)), dtype=np.float16)
    scales[0, 0] = 65504.0
    zeros = rng.integers(0, 16, (N, K // g)).astype(np.uint8)
    for mode in ("asym", "sym"):
        xhat = orc.dequantize_ref(packed, scales, zeros, g, mode)
        want = torch.from_numpy(xhat.astype(np.float32)).to(torch.float16).numpy()
        got = orc.dequantize_rounded_ref(packed, scales, zeros, g, mode, "f16")
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
        assert np.array_equal(np.isinf(got), np.abs(xhat) >= 65520.0)
