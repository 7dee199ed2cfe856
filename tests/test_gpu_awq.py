"""GPU parity of AWQ-style scaling against the CPU oracle (reading R9 of the oracle).

* q4_quantize_rtn_scaled and q4_scale_columns are bit-exact against the oracle given the same
  fp32 scales (taken from the oracle).
* q4_awq_search: the per-alpha errors agree with the oracle's within 2 % (the GPU's products
  are the library's bf16 W4A16 outputs, the oracle's are exact); the chosen alpha's oracle error
  is within that tolerance of the oracle's smallest; the chosen scales agree with the oracle's
  for that alpha to 1e-5 relative (fp32 log2 / exp2 against fp64); the final quantization is
  the library's scaled quantization of the returned scales; alpha = 0 (s = 1 exactly) reduces to
  plain RTN bit for bit; and two runs give identical outputs.
"""
import numpy as np
import pytest

from oracle import q4_oracle as orc
from synth import f64_to_bf16_bits

pytestmark = pytest.mark.gpu

ERR_RTOL = 0.02


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from tests.gpu_util import require_gpu
    require_gpu()


def _dev_bf16(bits):
    from tests.gpu_util import dev_bf16
    return dev_bf16(bits)


def _host_u16(t):
    from tests.gpu_util import host_u16
    return host_u16(t)


def _salient_layer(N, K, M, seed, n_salient=8, factor=30.0):
    rng = np.random.default_rng(seed)
    X = rng.normal(0, 1, (M, K))
    X[:, rng.choice(K, n_salient, replace=False)] *= factor
    W = rng.normal(0, 0.02, (N, K))
    W_bits = f64_to_bf16_bits(W)
    X_bits = f64_to_bf16_bits(X)
    Yref_bits = f64_to_bf16_bits(orc.bf16_bits_to_f32(X_bits).astype(np.float64) @
                                 orc.bf16_bits_to_f32(W_bits).astype(np.float64).T)
    return W_bits, X_bits, Yref_bits


def _same_quant(gpu, ref, label):
    import torch
    gp, gs, gz = gpu
    rp, rs, rz = ref
    for name, a, b in (("packed", gp.cpu().numpy(), rp), ("scales", _host_u16(gs), rs.view(np.uint16)),
                       ("zeros", gz.cpu().numpy(), rz)):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)[:5]
            raise AssertionError(f"{label}: {name} differs at {bad.tolist()}")


@pytest.mark.parametrize("N,K,g", [(64, 256, 32), (33, 1024, 128), (17, 480, 96), (8, 8192, 8192), (129, 2048, 64),
                                    (40, 4096, 32), (9, 1536, 512), (1030, 512, 256)])
@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_quantize_scaled_bitexact(N, K, g, mode):
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import log
    rng = np.random.default_rng(N + K + g)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    a = np.abs(rng.standard_normal(K)) + 0.05
    a[rng.choice(K, 4, replace=False)] *= 40
    for alpha in (0.0, 0.3, 1.0):
        s = orc.awq_scales_ref(a, alpha)
        got = q4.quantize_rtn_scaled(_dev_bf16(W_bits), torch.from_numpy(s).cuda(), g, mode)
        torch.cuda.synchronize()
        _same_quant(got, orc.quantize_rtn_scaled_ref(W_bits, s, g, mode), f"N={N} K={K} g={g} {mode} a={alpha}")
    log(f"scaled quantize parity ok: N={N} K={K} g={g} {mode}")


@pytest.mark.parametrize("rows,cols", [(1, 8), (5, 64), (37, 1000), (300, 4096), (2048, 8192)])
def test_scale_columns_bitexact(rows, cols):
    import torch
    import weight_only_int4_group_amd as q4
    rng = np.random.default_rng(rows * 3 + cols)
    A_bits = f64_to_bf16_bits(rng.normal(0, 1, (rows, cols)) * np.exp2(rng.integers(-30, 30, (rows, cols))))
    s = orc.awq_scales_ref(np.abs(rng.standard_normal(cols)) + 0.01, 0.7)
    sd = torch.from_numpy(s).cuda()
    for op in ("mul", "div"):
        out = q4.scale_columns(_dev_bf16(A_bits), sd, op)
        torch.cuda.synchronize()
        assert np.array_equal(_host_u16(out), orc.scale_columns_ref(A_bits, s, op)), op
    A = _dev_bf16(A_bits)
    q4.scale_columns_into(A, sd, "div", A)                 # in place
    torch.cuda.synchronize()
    assert np.array_equal(_host_u16(A), orc.scale_columns_ref(A_bits, s, "div"))


def _run_awq(W_bits, X_bits, Yref_bits, g, mode, n_alpha):
    import torch
    import weight_only_int4_group_amd as q4
    s, p, sc, z, err, best = q4.awq_search(_dev_bf16(X_bits), _dev_bf16(Yref_bits), _dev_bf16(W_bits), g,
                                           mode, n_alpha)
    torch.cuda.synchronize()
    return s, (p, sc, z), err.cpu().numpy(), int(best.cpu().numpy()[0])


@pytest.mark.parametrize("N,K,M,g,mode", [(256, 1024, 128, 128, "asym"), (192, 512, 96, 32, "sym"),
                                          (100, 768, 200, 64, "asym"), (64, 960, 64, 96, "asym")])
def test_awq_search_matches_oracle(N, K, M, g, mode):
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import log
    W_bits, X_bits, Yref_bits = _salient_layer(N, K, M, N + K + M + g)
    ref = orc.awq_search_ref(W_bits, X_bits, Yref_bits, g, mode, n_alpha=11)
    s, quant, err, best = _run_awq(W_bits, X_bits, Yref_bits, g, mode, 11)
    rel = np.abs(err - ref["errors"]) / ref["errors"]
    log(f"awq N={N} K={K} M={M} g={g} {mode}: gpu best {best} oracle best {ref['best']}, "
        f"max rel error difference {rel.max():.2e}")
    assert np.all(rel <= ERR_RTOL), rel
    assert 0 <= best < 11
    assert ref["errors"][best] <= ref["errors"].min() * (1 + 2 * ERR_RTOL)
    assert ref["best"] > 0 and ref["errors"][ref["best"]] < 0.9 * ref["errors"][0]    # the search helps
    s_host = s.cpu().numpy()
    want = ref["scales"][best].astype(np.float64)
    assert np.all(np.abs(s_host - want) <= 1e-5 * want)
    again = q4.quantize_rtn_scaled(_dev_bf16(W_bits), s, g, mode)
    torch.cuda.synchronize()
    for a, b in zip(quant, again):
        assert torch.equal(a, b)
    # identical outputs on a second run (fixed-order reductions)
    s2, quant2, err2, best2 = _run_awq(W_bits, X_bits, Yref_bits, g, mode, 11)
    assert best2 == best and np.array_equal(err2, err) and torch.equal(s2, s)
    for a, b in zip(quant2, quant):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_awq_search_alpha0_is_plain_rtn(mode):
    W_bits, X_bits, Yref_bits = _salient_layer(96, 512, 48, 11)
    s, quant, err, best = _run_awq(W_bits, X_bits, Yref_bits, 32, mode, 1)
    assert best == 0
    assert np.array_equal(s.cpu().numpy(), np.ones(512, np.float32))
    _same_quant(quant, orc.quantize_rtn_ref(W_bits, 32, mode), "alpha 0")
    ref = orc.awq_search_ref(W_bits, X_bits, Yref_bits, 32, mode, n_alpha=1)
    assert abs(err[0] - ref["errors"][0]) <= ERR_RTOL * ref["errors"][0]


def test_awq_search_zero_calibration_gives_unit_scales():
    """An all-zero calibration set: s = 1 for every alpha, all errors equal, index 0 chosen."""
    W_bits, X_bits, Yref_bits = _salient_layer(64, 256, 16, 12)
    X0 = np.zeros_like(X_bits)
    Y0 = np.zeros_like(Yref_bits)
    s, quant, err, best = _run_awq(W_bits, X0, Y0, 64, "asym", 5)
    assert best == 0 and np.all(err == 0.0)
    assert np.array_equal(s.cpu().numpy(), np.ones(256, np.float32))
    _same_quant(quant, orc.quantize_rtn_ref(W_bits, 64, "asym"), "zero calibration")
