"""Pins of the oracle's GPTQ (reading R11 of the oracle), CPU only.

* The pages' toy: the printed GPTQ output error and weight-space error.
* The library-format gptq_ref (Cholesky factor of H^-1) against the toy's route (closed-form
  updates on the trailing block of H) with the library's group quantizer: identical codes.
* Against an independent algebraic form written here: with H = Ut Ut^T (Ut upper triangular,
  the Cholesky factorisation of H in reversed order), the compensated weight of column i is
  w_i + sum_{j<i} (w_j - x_hat_j) Ut[j, i] / Ut[i, i] with the ORIGINAL w_j: identical codes.
* Special cases that reduce to RTN bit for bit: a diagonal Hessian (orthogonal calibration
  columns) and an all-zero calibration set; column 0 always takes its RTN code.
* GPTQ's objective: the calibration output error is below RTN's.
"""
import json
import os

import numpy as np
import pytest

from oracle import q4_oracle as orc
from synth import bf16_bits_to_f32, f64_to_bf16_bits
from tests.test_oracle_awq import toy_data

QMAX3 = 3


def toy_gptq(o):
    """(held-out output error, weight error, RTN weight error) of the toy with oracle module o."""
    W, xcal, xtest = toy_data()
    scales = np.abs(W).max(axis=1) / QMAX3
    quant_col = lambda i, v: np.clip(np.round(v / scales), -QMAX3 - 1, QMAX3) * scales
    Q = o.gptq_toy(W, xcal, quant_col)
    out = np.linalg.norm(xtest @ W.T - xtest @ Q.T) / np.linalg.norm(xtest @ W.T)
    Q_rtn = np.clip(np.round(W / scales[:, None]), -QMAX3 - 1, QMAX3) * scales[:, None]
    return out, np.linalg.norm(W - Q) / np.linalg.norm(W), np.linalg.norm(W - Q_rtn) / np.linalg.norm(W)


def _layer(N, K, M, seed, n_salient=4, factor=8.0):
    """Correlated calibration activations with a few large channels (the toy's structure)."""
    rng = np.random.default_rng(seed)
    mix = rng.normal(0, 1, (K, K)) / np.sqrt(K)
    fac = np.ones(K)
    fac[rng.choice(K, n_salient, replace=False)] = factor
    X = (rng.normal(0, 1, (M, K)) @ mix + 0.3 * rng.normal(0, 1, (M, K))) * fac
    W = rng.normal(0, 0.05, (N, K))
    return f64_to_bf16_bits(W), f64_to_bf16_bits(X)


def _group_params(W_bits, g, mode):
    _, s, z = orc.quantize_rtn_ref(W_bits, g, mode)
    return s.astype(np.float32), z.astype(np.int64)


def _code(v32, s32, z, mode):
    qmin, qmax = (0, 15) if mode == "asym" else (-8, 7)
    return int(np.clip(np.rint(np.float32(v32) / np.float32(s32)) + z, qmin, qmax))


def toy_route_codes(o, W_bits, X_bits, g, mode):
    """Codes of o.gptq_toy (closed-form updates on the trailing block of H) with the library's
    group quantizer."""
    s32, z = _group_params(W_bits, g, mode)
    X = bf16_bits_to_f32(X_bits).astype(np.float64)
    W = bf16_bits_to_f32(W_bits).astype(np.float64)
    N, K = W.shape
    codes = np.empty((N, K), dtype=np.int64)

    def quant_col(i, v):
        G = i // g
        codes[:, i] = [_code(np.float32(v[r]), s32[r, G], z[r, G], mode) for r in range(N)]
        return s32[:, G].astype(np.float64) * (codes[:, i] - z[:, G])

    o.gptq_toy(W, X, quant_col)
    return codes


def feedback_form_codes(W_bits, X_bits, g, mode, damp=0.01):
    """Independent route: reversed-order Cholesky of H and error feedback from the original
    weights (the form the GPU kernels use)."""
    X = bf16_bits_to_f32(X_bits).astype(np.float64)
    H = X.T @ X
    H = H + damp * np.mean(np.diag(H)) * np.eye(H.shape[0])
    rev = slice(None, None, -1)
    Ut = np.linalg.cholesky(H[rev][:, rev])[rev][:, rev]           # H = Ut Ut^T, Ut upper
    assert np.allclose(Ut @ Ut.T, H) and np.allclose(np.tril(Ut, -1), 0)
    T = Ut / np.diag(Ut)[None, :]
    s32, z = _group_params(W_bits, g, mode)
    W = bf16_bits_to_f32(W_bits).astype(np.float64)
    N, K = W.shape
    D = np.zeros((N, K))
    codes = np.empty((N, K), dtype=np.int64)
    for i in range(K):
        wp = W[:, i] + D[:, :i] @ T[:i, i]
        G = i // g
        for r in range(N):
            codes[r, i] = _code(np.float32(wp[r]), s32[r, G], z[r, G], mode)
        D[:, i] = W[:, i] - s32[:, G].astype(np.float64) * (codes[:, i] - z[:, G])
    return codes


def _ref_codes(o, W_bits, X_bits, g, mode):
    packed, _, _ = o.gptq_ref(W_bits, X_bits, g, mode)
    return o.unpack_codes_ref(packed, mode)


def test_toy_gptq_3bit(golden_dir):
    gt = json.load(open(os.path.join(golden_dir, "toy_gptq_3bit.json")))
    out, werr, rtn_werr = toy_gptq(orc)
    assert round(out, gt["output_decimals"]) == gt["gptq_output_error"]
    assert round(werr, gt["weight_decimals"]) == gt["gptq_weight_error"]
    assert round(rtn_werr, gt["weight_decimals"]) == gt["rtn_weight_error"]


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_gptq_ref_matches_toy_route(mode):
    W_bits, X_bits = _layer(12, 96, 300, 3)
    assert np.array_equal(_ref_codes(orc, W_bits, X_bits, 32, mode), toy_route_codes(orc, W_bits, X_bits, 32, mode))


@pytest.mark.parametrize("mode,g", [("asym", 32), ("sym", 64), ("asym", 128)])
def test_gptq_ref_matches_feedback_form(mode, g):
    W_bits, X_bits = _layer(20, 256, 512, 4)
    assert np.array_equal(_ref_codes(orc, W_bits, X_bits, g, mode), feedback_form_codes(W_bits, X_bits, g, mode))


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_gptq_diagonal_hessian_is_rtn(mode):
    """Calibration rows along the coordinate axes with distinct magnitudes: H is diagonal, the
    inverse has no off-diagonal entries, so nothing is compensated."""
    rng = np.random.default_rng(5)
    K = 64
    X = np.diag(np.exp2(rng.integers(-3, 4, K)).astype(np.float64))
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.05, (10, K)))
    got = orc.gptq_ref(W_bits, f64_to_bf16_bits(X), 32, mode)
    for a, b in zip(got, orc.quantize_rtn_ref(W_bits, 32, mode)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_gptq_zero_calibration_is_rtn(mode):
    W_bits, _ = _layer(8, 64, 16, 6)
    got = orc.gptq_ref(W_bits, np.zeros((16, 64), np.uint16), 32, mode)
    for a, b in zip(got, orc.quantize_rtn_ref(W_bits, 32, mode)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_gptq_scales_fixed_up_front_and_first_column_rtn(mode):
    W_bits, X_bits = _layer(16, 128, 256, 7)
    p, s, z = orc.gptq_ref(W_bits, X_bits, 64, mode)
    rp, rs, rz = orc.quantize_rtn_ref(W_bits, 64, mode)
    assert np.array_equal(s.view(np.uint16), rs.view(np.uint16)) and np.array_equal(z, rz)
    c, rc = orc.unpack_codes_ref(p, mode), orc.unpack_codes_ref(rp, mode)
    assert np.array_equal(c[:, 0], rc[:, 0])
    assert (c != rc).mean() > 0.05                       # the compensation does change codes


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_gptq_lowers_calibration_output_error(mode):
    W_bits, X_bits = _layer(32, 256, 512, 8)
    X = bf16_bits_to_f32(X_bits).astype(np.float64)
    W = bf16_bits_to_f32(W_bits).astype(np.float64)
    err = lambda q: np.linalg.norm(X @ W.T - X @ orc.dequantize_ref(*q, 32, mode).T)
    e_gptq = err(orc.gptq_ref(W_bits, X_bits, 32, mode))
    e_rtn = err(orc.quantize_rtn_ref(W_bits, 32, mode))
    assert e_gptq < 0.9 * e_rtn


def gptq_pins_hold(o) -> bool:
    """The pins above in compact form, for the planted-mistake tests."""
    gt = {"out": 0.2272, "w": 0.409}
    out, werr, _ = toy_gptq(o)
    if round(out, 4) != gt["out"] or round(werr, 3) != gt["w"]:
        return False
    W_bits, X_bits = _layer(12, 96, 300, 3)
    for mode in ("asym", "sym"):
        ref = _ref_codes(o, W_bits, X_bits, 32, mode)
        if not np.array_equal(ref, feedback_form_codes(W_bits, X_bits, 32, mode)):
            return False
        if not np.array_equal(ref, toy_route_codes(o, W_bits, X_bits, 32, mode)):
            return False
    rng = np.random.default_rng(5)
    X = np.diag(np.exp2(rng.integers(-3, 4, 64)).astype(np.float64))
    Wd = f64_to_bf16_bits(rng.normal(0, 0.05, (6, 64)))
    for a, b in zip(o.gptq_ref(Wd, f64_to_bf16_bits(X), 32, "asym"), orc.quantize_rtn_ref(Wd, 32, "asym")):
        if not np.array_equal(a, b):
            return False
    return True
