"""Pins of the oracle's W8A16 format (reading R10 of the oracle): the pages' W8A16 figures
with fp16 scales, storage and range rules, exact on-grid round trips and a brute-force
nearest-code search."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import q4_oracle as orc
from synth import f64_to_bf16_bits
from tests.test_oracle_pins import _granularity_tensors, _rel


def test_w8a16_granularity_with_fp16_scale(golden_dir):
    """'Granularity and outliers': per-channel symmetric INT8 weights give weight error 0.0078
    and W8A16 output error 0.0079; storing the scale as fp16 with fp32 arithmetic (the
    library's rule) leaves both printed figures unchanged."""
    gt = json.load(open(os.path.join(golden_dir, "granularity_table.json")))
    W, X = _granularity_tensors()
    q, s, _ = orc.quantize_groups(W.astype(np.float32).reshape(1024, 1, 1024), *orc.Q8_RANGE["sym"],
                                  "sym", "fp16", np.float32)
    Wq = (q * s.astype(np.float64)[..., None]).reshape(W.shape)
    d = gt["decimals"]
    assert round(_rel(W, Wq), d) == gt["weight_error"]["int8_per_channel"]
    assert round(_rel(X @ W.T, X @ Wq.T), d) == gt["output_error"]["weight_only_w8a16"]


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_quantize8_storage_and_ranges(mode):
    rng = np.random.default_rng(1)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.05, (40, 512)) * np.exp(rng.uniform(-3, 3, (40, 1))))
    codes, scales, zeros = orc.quantize8_rtn_ref(W_bits, 64, mode)
    assert codes.dtype == np.uint8 and codes.shape == (40, 512)
    assert scales.dtype == np.float16 and scales.shape == (40, 8)
    q = orc.codes8_ref(codes, mode)
    if mode == "sym":
        assert np.all(zeros == 0) and q.min() >= -127 and q.max() <= 127
        # the group's largest |x| maps to +-127
        x = orc.bf16_bits_to_f32(W_bits).reshape(40, 8, 64)
        i = np.abs(x).argmax(axis=-1)
        assert np.all(np.abs(np.take_along_axis(q.reshape(40, 8, 64), i[..., None], -1)) == 127)
        # two's complement storage
        assert np.array_equal(codes, (q & 0xFF).astype(np.uint8))
    else:
        assert q.min() >= 0 and q.max() <= 255 and zeros.max() <= 255
        # the group minimum maps to 0 (alpha <= 0 is the group minimum here)
        x = orc.bf16_bits_to_f32(W_bits).reshape(40, 8, 64)
        i = x.argmin(axis=-1)
        assert np.all(np.take_along_axis(q.reshape(40, 8, 64), i[..., None], -1) == 0)


def test_quantize8_on_grid_round_trip():
    """W already on a 2^-9 grid, s (q - z) with both code ends present: codes, zero-points and
    the dequantised weights are reproduced exactly."""
    rng = np.random.default_rng(2)
    N, K, g = 16, 512, 128
    G = K // g
    z = rng.integers(0, 256, (N, G))
    q = rng.integers(0, 256, (N, G, g))
    q[..., 0], q[..., 1] = 0, 255
    W = ((q - z[..., None]) * 2.0 ** -9).reshape(N, K)
    codes, scales, zeros = orc.quantize8_rtn_ref(f64_to_bf16_bits(W), g, "asym")
    assert np.array_equal(orc.dequantize8_ref(codes, scales, zeros, g, "asym"), W)
    assert np.all(scales.astype(np.float64) == 2.0 ** -9)


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_quantize8_brute_force_nearest(mode):
    """Each code is the grid point s (q - z) nearest to x (exact rationals), ties to even q - z,
    within the clip range."""
    rng = np.random.default_rng(3)
    W_bits = f64_to_bf16_bits(rng.normal(0, 1, (6, 64)))
    codes, scales, zeros = orc.quantize8_rtn_ref(W_bits, 32, mode)
    q = orc.codes8_ref(codes, mode)
    x = orc.bf16_bits_to_f32(W_bits)
    lo, hi = orc.Q8_RANGE[mode]
    for n in range(6):
        for k in range(64):
            s = Fraction(float(scales[n, k // 32]))
            zz = int(zeros[n, k // 32])
            xv = Fraction(float(x[n, k]))
            best = min(range(lo, hi + 1), key=lambda c: (abs(xv - s * (c - zz)), (c - zz) % 2))
            assert q[n, k] == best, (n, k)


def w8_pins_hold(o) -> bool:
    """The pins above in compact form (used by the mutation tests)."""
    rng = np.random.default_rng(2)
    N, K, g = 16, 512, 128
    G = K // g
    z = rng.integers(0, 256, (N, G))
    q = rng.integers(0, 256, (N, G, g))
    q[..., 0], q[..., 1] = 0, 255
    W = ((q - z[..., None]) * 2.0 ** -9).reshape(N, K)
    codes, scales, zeros = o.quantize8_rtn_ref(f64_to_bf16_bits(W), g, "asym")
    if not np.array_equal(o.dequantize8_ref(codes, scales, zeros, g, "asym"), W):
        return False
    rng = np.random.default_rng(1)
    Wb = f64_to_bf16_bits(rng.normal(0, 0.05, (8, 128)))
    c, s, zz = o.quantize8_rtn_ref(Wb, 64, "sym")
    qq = o.codes8_ref(c, "sym")
    return int(np.abs(qq).max()) == 127 and np.array_equal(c, (qq & 0xFF).astype(np.uint8))
