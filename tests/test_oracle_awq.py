"""Pins of the oracle's AWQ-style scaling (reading R9 of the oracle) against the pages and
against independent routines: the pages' printed toy result, torch's fp32 arithmetic and
bf16 conversion, and closed forms of the scale rule."""
import json
import os

import numpy as np
import pytest

from oracle import q4_oracle as orc
from synth import f64_to_bf16_bits
from tests.test_oracle_pins import _qdq_sym


def toy_data():
    """The toy's activations and weights, drawn in the page's order (default_rng(1))."""
    rng = np.random.default_rng(1)
    d, rows, n = 128, 64, 1024
    mix = rng.normal(0, 1, (d, d)) / np.sqrt(d)
    factors = np.ones(d)
    factors[rng.choice(d, 4, replace=False)] = 8.0

    def acts(m):
        a = rng.normal(0, 1, (m, d)) @ mix
        b = 0.3 * rng.normal(0, 1, (m, d))
        return (a + b) * factors

    xcal = acts(n)
    xtest = acts(n)
    W = rng.normal(0, 0.05, (rows, d))
    return W, xcal, xtest


def toy_awq(o):
    """(alpha, held-out relative output error) of the toy's AWQ with oracle module o."""
    W, xcal, xtest = toy_data()
    Q, alpha, _ = o.awq_toy(W, xcal, lambda w: _qdq_sym(w, 3, (W.shape[0], 1, W.shape[1])))
    err = np.linalg.norm(xtest @ W.T - xtest @ Q.T) / np.linalg.norm(xtest @ W.T)
    return alpha, err


def test_toy_awq_3bit(golden_dir):
    gt = json.load(open(os.path.join(golden_dir, "toy_awq_3bit.json")))
    alpha, err = toy_awq(orc)
    assert round(alpha, gt["alpha_decimals"]) == gt["alpha"]
    assert round(err, gt["output_decimals"]) == gt["output_error"]


def _torch_f32_bf16(x32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_f32_to_bf16_matches_torch():
    """Against torch's fp32 -> bf16 conversion (round half to even) over normal and subnormal
    values, exact ties, and values that round past bf16's largest finite value."""
    rng = np.random.default_rng(3)
    with np.errstate(over="ignore"):
        x = (rng.standard_normal(100000) * np.exp2(rng.uniform(-149, 127, 100000))).astype(np.float32)
    x = x[np.isfinite(x)]
    bits = rng.integers(0, 2 ** 31, 20000, dtype=np.uint64).astype(np.uint32)
    ties = ((bits & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32)     # exactly halfway
    ties = ties[np.isfinite(ties)]
    big = np.array([3.3895e38, 3.39e38, 3.4e38, -3.4e38, 1e-45, -1e-45, 0.0, -0.0], np.float32)
    for v in (x, ties, big):
        assert np.array_equal(orc.f32_to_bf16_bits_ref(v), _torch_f32_bf16(v))


def test_awq_scales_closed_forms():
    rng = np.random.default_rng(4)
    a = np.abs(rng.standard_normal(512)) + 0.01
    assert np.array_equal(orc.awq_scales_ref(a, 0.0), np.ones(512, np.float32))
    for alpha in (0.1, 0.3, 0.5, 1.0):
        s = orc.awq_scales_ref(a, alpha).astype(np.float64)
        # geometric normalisation: the largest and smallest scale multiply to 1
        assert abs(s.max() * s.min() - 1.0) < 4e-7
        # s_j / s_k = (a_j / a_k)^alpha
        i, j = int(np.argmax(a)), int(np.argmin(a))
        assert abs(s[i] / s[j] - (a[i] / a[j]) ** alpha) < 1e-5 * (a[i] / a[j]) ** alpha
        assert np.all(np.diff(s[np.argsort(a)]) >= 0)          # monotone in a
    # alpha = 1: s = a / sqrt(max a min a)
    s1 = orc.awq_scales_ref(a, 1.0)
    assert np.allclose(s1, a / np.sqrt(a.max() * a.min()), rtol=1e-6, atol=0)


def test_awq_scales_degenerate_channels():
    a = np.array([0.0, 1.0, 4.0, 0.0])
    s = orc.awq_scales_ref(a, 0.5).astype(np.float64)
    floor = 2.0 ** -20 * 4.0
    want = np.sqrt(np.array([floor, 1.0, 4.0, floor]))
    want = want / np.sqrt(want.max() * want.min())
    assert np.allclose(s, want, rtol=1e-6)
    assert np.array_equal(orc.awq_scales_ref(np.zeros(5), 0.7), np.ones(5, np.float32))


def test_scale_columns_matches_torch():
    """bf16(fl32(A * s)) and bf16(fl32(A / s)) against torch's fp32 product / quotient."""
    import torch
    rng = np.random.default_rng(5)
    A_bits = f64_to_bf16_bits(rng.normal(0, 1, (37, 96)) * np.exp2(rng.integers(-20, 20, (37, 96))))
    s = (np.abs(rng.standard_normal(96)) * 3 + 0.05).astype(np.float32)
    A = torch.from_numpy(A_bits.view(np.int16)).view(torch.bfloat16).float()
    st = torch.from_numpy(s)
    mul = (A * st).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    div = (A / st).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.scale_columns_ref(A_bits, s, "mul"), mul)
    assert np.array_equal(orc.scale_columns_ref(A_bits, s, "div"), div)
    # power-of-two scales only move exponents: exact both ways
    p2 = np.exp2(rng.integers(-8, 8, 96)).astype(np.float32)
    back = orc.scale_columns_ref(orc.scale_columns_ref(A_bits, p2, "mul"), p2, "div")
    assert np.array_equal(back, A_bits)


def _salient_layer(N=64, K=256, M=96, seed=6):
    """Gaussian layer whose activations have a few large channels (the toy's structure)."""
    rng = np.random.default_rng(seed)
    X = rng.normal(0, 1, (M, K))
    X[:, rng.choice(K, 4, replace=False)] *= 30.0
    W = rng.normal(0, 0.05, (N, K))
    W_bits = f64_to_bf16_bits(W)
    X_bits = f64_to_bf16_bits(X)
    Yref_bits = f64_to_bf16_bits(orc.bf16_bits_to_f32(X_bits).astype(np.float64) @
                                 orc.bf16_bits_to_f32(W_bits).astype(np.float64).T)
    return W_bits, X_bits, Yref_bits


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_awq_search_alpha0_is_plain_rtn(mode):
    """alpha = 0 gives s = 1: the weights are quantized exactly as plain RTN and the error is
    plain RTN's output error."""
    W_bits, X_bits, Yref_bits = _salient_layer()
    r = orc.awq_search_ref(W_bits, X_bits, Yref_bits, 32, mode, n_alpha=1)
    assert r["best"] == 0 and r["alphas"] == [0.0]
    assert np.array_equal(r["scales"][0], np.ones(W_bits.shape[1], np.float32))
    plain = orc.quantize_rtn_ref(W_bits, 32, mode)
    for a, b in zip(r["quant"], plain):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    Y, _ = orc.matmul_ref(X_bits, *plain, 32, mode)
    err = ((Y - orc.bf16_bits_to_f32(Yref_bits).astype(np.float64)) ** 2).sum()
    assert r["errors"][0] == err


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_awq_search_beats_rtn_on_salient_channels(mode):
    """The pages' claim for activation-aware scaling: with a few large activation channels the
    searched alpha gives a smaller output error than plain RTN (alpha = 0)."""
    W_bits, X_bits, Yref_bits = _salient_layer()
    r = orc.awq_search_ref(W_bits, X_bits, Yref_bits, 128, mode, n_alpha=11)
    assert r["alphas"] == [i / 10 for i in range(11)]
    assert r["best"] == int(np.argmin(r["errors"])) and r["best"] > 0
    assert r["errors"][r["best"]] < 0.9 * r["errors"][0]
    assert np.array_equal(r["absmean"], np.abs(orc.bf16_bits_to_f32(X_bits).astype(np.float64)).mean(axis=0))


@pytest.mark.parametrize("mode,g,seed", [("asym", 128, 6), ("sym", 32, 9), ("asym", 64, 11)])
def test_awq_search_ref_picks_the_toy_search_alpha(mode, g, seed):
    """The library-format search (fp32 scales, bf16(W s) and bf16(X / s), squared error against
    a bf16 reference) and the toy's search (fp64, 1/s folded onto the weights, exact products)
    run with the library's group quantizer pick the same alpha on layers with salient
    channels."""
    W_bits, X_bits, Yref_bits = _salient_layer(seed=seed)
    r = orc.awq_search_ref(W_bits, X_bits, Yref_bits, g, mode, n_alpha=11)

    def qdq(ws):
        q = orc.quantize_rtn_ref(f64_to_bf16_bits(ws), g, mode)
        return orc.dequantize_ref(*q, g, mode)

    W = orc.bf16_bits_to_f32(W_bits).astype(np.float64)
    X = orc.bf16_bits_to_f32(X_bits).astype(np.float64)
    _, alpha, scores = orc.awq_toy(W, X, qdq)
    assert r["best"] > 0
    assert r["alphas"][r["best"]] == alpha
    # the two scorings agree on the shape of the curve, not only on its minimum
    ratio = np.sqrt(r["errors"]) / scores
    assert ratio.max() / ratio.min() < 1.2


def test_awq_toy_equal_channels_first_alpha_wins():
    """Channels of equal mean magnitude give s = 1 for every alpha, so every candidate scores the
    same and the first alpha of the grid (0) must win."""
    rng = np.random.default_rng(12)
    X = rng.choice([-1.0, 1.0], size=(40, 64))
    W = rng.normal(0, 0.05, (8, 64))
    _, alpha, scores = orc.awq_toy(W, X, lambda w: _qdq_sym(w, 3, (8, 1, 64)))
    assert np.all(scores == scores[0]) and alpha == 0.0


def awq_pins_hold(o) -> bool:
    """The pins above in compact form (used by the mutation tests)."""
    alpha, err = toy_awq(o)
    if round(alpha, 1) != 0.3 or round(err, 4) != 0.2128:
        return False
    rng = np.random.default_rng(12)
    Xe = rng.choice([-1.0, 1.0], size=(40, 64))
    We = rng.normal(0, 0.05, (8, 64))
    if o.awq_toy(We, Xe, lambda w: _qdq_sym(w, 3, (8, 1, 64)))[1] != 0.0:
        return False
    rng = np.random.default_rng(4)
    a = np.abs(rng.standard_normal(512)) + 0.01
    s = o.awq_scales_ref(a, 0.5).astype(np.float64)
    if abs(s.max() * s.min() - 1.0) > 4e-7:
        return False
    x = (rng.standard_normal(5000) * np.exp2(rng.uniform(-140, 120, 5000))).astype(np.float32)
    if not np.array_equal(o.f32_to_bf16_bits_ref(x), _torch_f32_bf16(x)):
        return False
    W_bits, X_bits, Yref_bits = _salient_layer()
    r = o.awq_search_ref(W_bits, X_bits, Yref_bits, 128, "asym", n_alpha=11)
    if not (r["alphas"][-1] == 1.0 and 0 < r["best"] and r["errors"][r["best"]] < 0.9 * r["errors"][0]):
        return False

    def qdq(ws):
        q = o.quantize_rtn_ref(f64_to_bf16_bits(ws), 128, "asym")
        return o.dequantize_ref(*q, 128, "asym")

    _, alpha, _ = o.awq_toy(o.bf16_bits_to_f32(W_bits).astype(np.float64),
                            o.bf16_bits_to_f32(X_bits).astype(np.float64), qdq)
    return r["alphas"][r["best"]] == alpha
