"""Properties that pin the oracle to the mathematics rather than to itself.

* exact rational recomputation: the scale, zero-point and codes recomputed from the
  formulas of "DL S067 · Quantization", §1 with exact fractions and an explicit IEEE
  round-to-nearest-even written here (not numpy's);
* brute force: every code is a nearest grid point of the stored (scale, zero), ties to an
  even distance from z;
* invariants: |x - x_hat| <= scale/2 where unclipped, z = 0 and q in [-7, 7] in symmetric
  mode, x = 0 maps exactly to 0, codes are monotone within a group;
* on-grid round trip: weights that already lie on a 2^-6 grid come back unchanged;
* matmul: exact-fraction dot products, linearity, all-ones rows give row sums.
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

from oracle import q4_oracle as orc
from synth import f64_to_bf16_bits

SETTINGS = settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])


# --------------------------------------------------------------------- exact IEEE rounding
def round_ieee(v: Fraction, precision: int, emin: int, emax: int) -> Fraction:
    """Round a rational to the nearest binary float (ties to even), with subnormals.

    precision counts the leading bit (fp32: 24, fp16: 11); emin/emax are the normal
    exponent limits (fp32: -126/127, fp16: -14/15).  Overflow returns +-inf as a float.
    """
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - precision + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        return Fraction(sign) * Fraction(10) ** 400   # stands for inf
    return sign * r


def rn32(v):
    return round_ieee(v, 24, -126, 127)


def rn16(v):
    return round_ieee(v, 11, -14, 15)


def rne_int(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def exact_group(xs, mode):
    """Scale, zero-point and codes of one group, in exact rationals (readings R1-R5)."""
    xs = [Fraction(float(v)) for v in xs]
    if mode == "asym":
        lo, hi, qmin, qmax = min(min(xs), 0), max(max(xs), 0), 0, 15
        s32 = rn32(rn32(hi - lo) / 15)
    else:
        m, qmin, qmax = max(abs(v) for v in xs), -8, 7
        s32 = rn32(m / 7)
    s32 = min(s32, Fraction(65504))
    s16 = rn16(s32)
    if s16 == 0:
        s16 = Fraction(1)
    z = 0 if mode == "sym" else min(max(rne_int(-lo / s16), 0), 15)
    q = [min(max(rne_int(v / s16) + z, qmin), qmax) for v in xs]
    return s16, z, q


# --------------------------------------------------------------------- strategies
def _bf16_group(values):
    return orc.bf16_bits_to_f32(f64_to_bf16_bits(np.asarray(values, dtype=np.float64)))


magnitudes = st.sampled_from([1e-30, 1e-8, 1e-3, 0.02, 1.0, 300.0, 1e6, 1e30])


@st.composite
def random_groups(draw, g):
    kind = draw(st.sampled_from(["normal", "positive", "negative", "constant", "zeros",
                                 "sparse", "tiny", "halfgrid"]))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    mag = draw(magnitudes)
    if kind == "normal":
        v = rng.normal(0, mag, g)
    elif kind == "positive":
        v = np.abs(rng.normal(0, mag, g)) + mag * 0.1
    elif kind == "negative":
        v = -np.abs(rng.normal(0, mag, g)) - mag * 0.1
    elif kind == "constant":
        v = np.full(g, rng.normal(0, mag))
    elif kind == "zeros":
        v = np.zeros(g)
    elif kind == "sparse":
        v = np.zeros(g)
        v[rng.integers(0, g, 2)] = rng.normal(0, mag, 2)
    elif kind == "tiny":                       # values whose fp16 scale underflows
        v = rng.normal(0, 1e-12, g)
    else:                                      # exact ties: half-integer multiples of 2^e
        e = int(rng.integers(-20, 10))
        z = int(rng.integers(0, 16))
        idx = rng.integers(0, 30, g) / 2.0 - z
        idx[0], idx[1] = -z, 15 - z
        v = np.clip(idx, -z, 15 - z) * 2.0 ** e
    return _bf16_group(v)


# --------------------------------------------------------------------- exact recomputation
@SETTINGS
@given(st.sampled_from(["asym", "sym"]), st.sampled_from([8, 32, 128]), st.data())
def test_oracle_matches_exact_rationals(mode, g, data):
    x = data.draw(random_groups(g))
    qmin, qmax = (0, 15) if mode == "asym" else (-8, 7)
    q, s16, z = orc.quantize_groups(x[None, :], qmin, qmax, mode)
    es, ez, eq = exact_group(x, mode)
    assert Fraction(float(s16[0])) == es
    assert int(z[0]) == ez
    assert q[0].tolist() == eq


# --------------------------------------------------------------------- brute force
@SETTINGS
@given(st.sampled_from(["asym", "sym"]), st.data())
def test_codes_are_nearest_grid_points(mode, data):
    g = data.draw(st.sampled_from([4, 8]))
    x = data.draw(random_groups(g))
    qmin, qmax = (0, 15) if mode == "asym" else (-8, 7)
    q, s16, z = orc.quantize_groups(x[None, :], qmin, qmax, mode)
    s = Fraction(float(s16[0]))
    zz = int(z[0])
    for xv, qv in zip(x, q[0]):
        xf = Fraction(float(xv))
        dist = {c: abs(xf - s * (c - zz)) for c in range(qmin, qmax + 1)}
        best = min(dist.values())
        assert dist[int(qv)] == best
        ties = [c for c, d in dist.items() if d == best]
        if len(ties) > 1:
            assert (int(qv) - zz) % 2 == 0


# --------------------------------------------------------------------- invariants
@SETTINGS
@given(st.sampled_from(["asym", "sym"]), st.sampled_from([32, 64, 128]), st.data())
def test_invariants(mode, g, data):
    x = data.draw(random_groups(g))
    qmin, qmax = (0, 15) if mode == "asym" else (-8, 7)
    q, s16, z = orc.quantize_groups(x[None, :], qmin, qmax, mode)
    s = float(s16[0]); zz = int(z[0]); qq = q[0]
    xd = x.astype(np.float64)
    xhat = s * (qq - zz)
    spread = (max(xd.max(), 0) - min(xd.min(), 0)) / 15 if mode == "asym" else np.abs(xd).max() / 7
    saturated = spread > 65504
    normal_scale = 2.0 ** -14 <= spread <= 65504        # fp16 scale keeps 11 significant bits
    unclipped = (qq > qmin) & (qq < qmax)
    if not saturated:
        assert np.all(np.abs(xd - xhat)[unclipped] <= s / 2 * (1 + 2 ** -20))
    assert np.all(np.diff(qq[np.argsort(xd, kind="stable")]) >= 0)       # monotone
    if mode == "sym":
        assert zz == 0
        if normal_scale:
            assert qq.min() >= -7 and qq.max() <= 7                       # -8 never occurs
        if normal_scale:
            assert np.abs(qq).max() == 7                                  # absmax -> +-7
    else:
        assert 0 <= zz <= 15
        if normal_scale:
            assert np.all(np.abs(xd - xhat) <= s * (0.5 + 15 * 2 ** -11))
        if xd.min() < 0:
            assert qq[np.argmin(xd)] == 0                                 # minimum -> code 0
    zero_pos = xd == 0
    assert np.all(xhat[zero_pos] == 0)                                     # 0 exactly representable


def test_saturated_and_degenerate_groups():
    x = _bf16_group([3e38, -1.0] + [0.0] * 30)
    q, s16, z = orc.quantize_groups(x[None, :], 0, 15, "asym")
    assert float(s16[0]) == 65504.0 and q[0, 0] == 15
    x = _bf16_group([0.0] * 32)
    q, s16, z = orc.quantize_groups(x[None, :], 0, 15, "asym")
    assert float(s16[0]) == 1.0 and int(z[0]) == 0 and np.all(q == 0)
    x = _bf16_group([1e-10] * 32)
    q, s16, z = orc.quantize_groups(x[None, :], -8, 7, "sym")
    assert float(s16[0]) == 1.0 and np.all(q == 0)
    with pytest.raises(ValueError):
        orc.quantize_groups(np.array([[np.nan, 1.0]], np.float32), 0, 15, "asym")


# --------------------------------------------------------------------- on-grid round trip
@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_on_grid_round_trip(mode):
    rng = np.random.default_rng(11)
    N, K, g = 16, 256, 64
    G = K // g
    if mode == "asym":
        z = rng.integers(0, 16, (N, G))
        q = rng.integers(0, 16, (N, G, g))
        q[..., 0], q[..., 1] = 0, 15
        W = (q - z[..., None]) * 2.0 ** -6
    else:
        z = np.zeros((N, G), np.int64)
        q = rng.integers(-7, 8, (N, G, g))
        q[..., 0] = 7
        W = q * 2.0 ** -6
    W_bits = f64_to_bf16_bits(W.reshape(N, K))
    packed, scales, zeros = orc.quantize_rtn_ref(W_bits, g, mode)
    assert np.all(scales == np.float16(2.0 ** -6))
    assert np.array_equal(zeros.astype(np.int64), z)
    assert np.array_equal(orc.unpack_codes_ref(packed, mode).reshape(N, G, g), q)
    What = orc.dequantize_ref(packed, scales, zeros, g, mode)
    assert np.array_equal(What, W.reshape(N, K))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (5, K)))
    X = orc.bf16_bits_to_f32(X_bits).astype(np.float64)
    Y, A = orc.matmul_ref(X_bits, packed, scales, zeros, g, mode)
    W2 = W.reshape(N, K)
    Yt = np.array([[sum(Fraction(float(X[m, k])) * Fraction(float(W2[n, k])) for k in range(K))
                    for n in range(N)] for m in range(5)], dtype=object)
    assert np.all(np.abs(Y - Yt.astype(np.float64)) <= 1e-12 * A)


# --------------------------------------------------------------------- matmul pins
def test_matmul_exact_fractions_and_linearity():
    rng = np.random.default_rng(3)
    N, K, g, M = 5, 64, 32, 3
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        packed, scales, zeros = orc.quantize_rtn_ref(W_bits, g, mode)
        codes = orc.unpack_codes_ref(packed, mode)
        Y, A = orc.matmul_ref(X_bits, packed, scales, zeros, g, mode)
        X = orc.bf16_bits_to_f32(X_bits)
        for m in range(M):
            for n in range(N):
                acc = Fraction(0); aa = Fraction(0)
                for k in range(K):
                    zz = 0 if mode == "sym" else int(zeros[n, k // g])
                    w = Fraction(float(scales[n, k // g])) * (int(codes[n, k]) - zz)
                    acc += Fraction(float(X[m, k])) * w
                    aa += abs(Fraction(float(X[m, k])) * w)
                assert abs(Fraction(Y[m, n]) - acc) <= Fraction(K) * Fraction(2) ** -52 * aa
                assert abs(Fraction(A[m, n]) - aa) <= Fraction(K) * Fraction(2) ** -52 * aa
        # linearity in X and all-ones rows give row sums of x_hat
        X2_bits = f64_to_bf16_bits(2.0 * orc.bf16_bits_to_f32(X_bits))
        Y2, _ = orc.matmul_ref(X2_bits, packed, scales, zeros, g, mode)
        assert np.array_equal(Y2, 2.0 * Y)
        ones = f64_to_bf16_bits(np.ones((1, K)))
        Y1, _ = orc.matmul_ref(ones, packed, scales, zeros, g, mode)
        What = orc.dequantize_ref(packed, scales, zeros, g, mode)
        assert np.allclose(Y1[0], What.sum(axis=1), rtol=0, atol=1e-15)


def test_entries_ref_agrees_with_full():
    rng = np.random.default_rng(4)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (40, 128)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (7, 128)))
    packed, scales, zeros = orc.quantize_rtn_ref(W_bits, 32, "asym")
    Y, A = orc.matmul_ref(X_bits, packed, scales, zeros, 32, "asym")
    mi = rng.integers(0, 7, 30); ni = rng.integers(0, 40, 30)
    Ye, Ae = orc.matmul_entries_ref(X_bits, packed, scales, zeros, 32, "asym", mi, ni)
    assert np.allclose(Ye, Y[mi, ni], rtol=1e-13, atol=0)
    assert np.allclose(Ae, A[mi, ni], rtol=1e-13, atol=0)


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(8)
    for mode in ("asym", "sym"):
        W_bits = f64_to_bf16_bits(rng.normal(0, 1, (3, 96)))
        packed, scales, zeros = orc.quantize_rtn_ref(W_bits, 32, mode)
        codes = orc.unpack_codes_ref(packed, mode)
        lo = codes[:, 0::2] & 0xF
        hi = codes[:, 1::2] & 0xF
        assert np.array_equal((lo | (hi << 4)).astype(np.uint8), packed)
