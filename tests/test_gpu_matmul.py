"""GPU W4A16 matmul parity against the CPU oracle.

Inputs are quantized by the oracle on the host (never by the GPU), uploaded, multiplied on
the GPU through the C ABI, and every element (or, at full size, a sample of elements) must
satisfy |Y - Y_ref| <= 8e-3 * sum_k |X[m,k] * x_hat[n,k]| + 1e-6, Y_ref in fp64.
"""
import numpy as np
import pytest

from oracle import q4_oracle as orc
from synth import CONFIGS, f64_to_bf16_bits, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from tests.gpu_util import require_gpu
    require_gpu()


def kernels_for(M, N, K, g):
    """Every kernel that can run this shape (mirrors the rules stated in include/q4.h)."""
    ks = ["auto", "gemm"]
    if (M == 1 and K <= 16384) or (M == 2 and K <= 4096):
        ks.append("gemv")
    lds = 2 * M * K + 64 * (K // min(g, 128)) + 8192
    if 1 <= M <= 16 and (g in (32, 64) or g % 128 == 0) and lds <= 160 * 1024:
        ks.append("decode")
    return tuple(ks)


def _upload(packed, scales, zeros):
    from tests.gpu_util import dev
    return dev(packed), dev(scales.view(np.uint16)).view(__import__("torch").float16), dev(zeros)


def _gpu_matmul(X_bits, qw, g, mode, kernel="auto"):
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import dev_bf16, host_bf16_to_f64
    p, s, z = qw
    Y = q4.matmul(dev_bf16(X_bits), p, s, z, g, mode, kernel)
    torch.cuda.synchronize()
    return host_bf16_to_f64(Y)


def _check_full(X_bits, W_bits, g, mode, label, kernels=("auto",), quant=None):
    from tests.gpu_util import log
    packed, scales, zeros = quant if quant is not None else orc.quantize_rtn_ref(W_bits, g, mode)
    Y_ref, A = orc.matmul_ref(X_bits, packed, scales, zeros, g, mode)
    qw = _upload(packed, scales, zeros)
    for kernel in kernels:
        Y = _gpu_matmul(X_bits, qw, g, mode, kernel)
        ok, usage = orc.check_matmul(Y, Y_ref, A)
        log(f"matmul parity {label} kernel={kernel} M={X_bits.shape[0]} N={packed.shape[0]} "
            f"K={X_bits.shape[1]} g={g} {mode}: max tolerance usage {usage:.3e}")
        assert ok, f"{label} kernel={kernel}: tolerance exceeded (usage {usage})"
    return Y


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_configs_full(idx):
    cfg = CONFIGS[idx]
    W_bits, X_bits = make_layer(cfg)
    kernels = kernels_for(X_bits.shape[0], cfg.N, cfg.K, cfg.g)
    _check_full(X_bits, W_bits, cfg.g, cfg.mode, cfg.name, kernels)


def _check_sampled(X_bits, qw_host, g, mode, label, n_samples=4096, kernel="auto", seed=0):
    from tests.gpu_util import log
    packed, scales, zeros = qw_host
    Y = _gpu_matmul(X_bits, _upload(packed, scales, zeros), g, mode, kernel)
    M, N = Y.shape
    rng = np.random.default_rng(seed)
    mi = rng.integers(0, M, n_samples)
    ni = rng.integers(0, N, n_samples)
    mi = np.concatenate([mi, [0, M - 1, 0, M - 1]])
    ni = np.concatenate([ni, [0, 0, N - 1, N - 1]])
    Y_ref, A = orc.matmul_entries_ref(X_bits, packed, scales, zeros, g, mode, mi, ni)
    ok, usage = orc.check_matmul(Y[mi, ni], Y_ref, A)
    log(f"matmul parity (sampled) {label} kernel={kernel} M={M} N={N} g={g} {mode}: "
        f"max tolerance usage {usage:.3e}")
    assert ok, f"{label}: tolerance exceeded (usage {usage})"


@pytest.fixture(scope="module")
def layer70b():
    cfg = CONFIGS[3]
    W_bits, X_bits = make_layer(cfg)
    return cfg, X_bits, orc.quantize_rtn_ref(W_bits, cfg.g, cfg.mode)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_70b_mlp_decode(layer70b, M):
    cfg, X_bits, qw = layer70b
    for kernel in kernels_for(M, cfg.N, cfg.K, cfg.g):
        _check_sampled(X_bits[:M], qw, cfg.g, cfg.mode, cfg.name, n_samples=3000, kernel=kernel)


@pytest.mark.parametrize("g", [128, 32])
def test_prefill(g):
    cfg = CONFIGS[4]
    W_bits, X_bits = make_layer(cfg)
    qw = orc.quantize_rtn_ref(W_bits, g, cfg.mode)
    _check_sampled(X_bits, qw, g, cfg.mode, cfg.name, n_samples=4096)


@pytest.mark.parametrize("M,N,K,g", [(512, 64, 128, 128), (513, 300, 256, 32), (640, 256, 384, 128),
                                     (1000, 520, 512, 64), (700, 1030, 1024, 256), (777, 136, 640, 128)])
def test_prefill_ragged(M, N, K, g):
    """Large-M shapes on the LDS-staged GEMM: ragged M and N tiles, odd step counts, every g."""
    rng = np.random.default_rng(M + 3 * N + 7 * K + g)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full(X_bits, W_bits, g, mode, "prefill-ragged", ("auto", "gemm"))


@pytest.mark.parametrize("M,N,K,g", [(589, 22000, 384, 128), (512, 32768, 256, 32),
                                     (1024, 16384, 512, 256), (600, 21800, 640, 64)])
def test_prefill_large_tiles(M, N, K, g):
    """Shapes with at least as many 256 x 256 tiles as a 256-CU device has compute units, so
    the GEMM takes its 256-row tile: ragged M and N, odd and even step counts, every g."""
    import torch
    from tests.gpu_util import log
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-M // 256) * -(-N // 256)
    log(f"large-tile case M={M} N={N} K={K} g={g}: {tiles} tiles on {cus} compute units")
    rng = np.random.default_rng(M + N + K + g)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full(X_bits, W_bits, g, mode, "prefill-large", ("auto",))


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 13, 16, 17, 33, 64, 65, 129, 257])
@pytest.mark.parametrize("N,K,g", [(100, 96, 32), (37, 256, 64), (128, 4096, 128), (1, 32, 32),
                                   (50, 640, 128), (33, 1024, 256), (20, 8192, 8192)])
def test_ragged(M, N, K, g):
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full(X_bits, W_bits, g, mode, "ragged", kernels_for(M, N, K, g))


def test_special_values():
    rng = np.random.default_rng(7)
    N, K, g = 48, 512, 128
    W = rng.normal(0, 0.02, (N, K))
    W[0] = 0.0                                   # all-zero row: Y must be exactly 0
    W[1, :128] = 0.0                             # one all-zero group
    W[2] = 0.5                                   # constant row
    W[3] = np.abs(W[3])                          # all positive
    W[4] = 1e-10                                 # scale underflow -> 1.0
    W_bits = f64_to_bf16_bits(W)
    X = rng.normal(0, 1, (6, K))
    X[1] = 0.0                                   # all-zero activation row
    X[2, :] = 1e-20; X[2, ::7] = 1e20            # huge dynamic range within a row
    X[3] = 1.0                                   # all ones -> row sums
    X[4, :] = 0.0; X[4, 5] = 1.0                 # one-hot
    X_bits = f64_to_bf16_bits(X)
    for mode in ("asym", "sym"):
        for M in (1, 2, 6):
            Y = _check_full(X_bits[:M], W_bits, g, mode, "special", kernels_for(M, N, K, g))
            assert np.all(Y[:, 0] == 0.0)


def test_on_grid_weights_match_exact_product():
    """W already on a 2^-6 grid: the quantizer reproduces it, so Y must match X W^T."""
    rng = np.random.default_rng(21)
    N, K, g = 64, 1024, 128
    G = K // g
    z = rng.integers(0, 16, (N, G))
    q = rng.integers(0, 16, (N, G, g)); q[..., 0], q[..., 1] = 0, 15
    W = ((q - z[..., None]) * 2.0 ** -6).reshape(N, K)
    W_bits = f64_to_bf16_bits(W)
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (20, K)))
    packed, scales, zeros = orc.quantize_rtn_ref(W_bits, g, "asym")
    assert np.array_equal(orc.dequantize_ref(packed, scales, zeros, g, "asym"), W)
    X = orc.bf16_bits_to_f32(X_bits).astype(np.float64)
    exact = X @ W.T
    A = np.abs(X) @ np.abs(W).T
    for M in (1, 2, 7, 16, 20):
        for kernel in kernels_for(M, N, K, g):
            Y = _gpu_matmul(X_bits[:M], _upload(packed, scales, zeros), g, "asym", kernel)
            assert np.all(np.abs(Y - exact[:M]) <= orc.tol_ref(A[:M])), kernel


def test_m0_is_noop_and_nondefault_stream():
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import dev_bf16, host_bf16_to_f64
    rng = np.random.default_rng(3)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (64, 256)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (3, 256)))
    packed, scales, zeros = orc.quantize_rtn_ref(W_bits, 64, "asym")
    p, s, z = _upload(packed, scales, zeros)
    Y0 = torch.full((0, 64), 1.0, dtype=torch.bfloat16, device="cuda")
    q4.matmul_into(dev_bf16(X_bits[:0]), p, s, z, 64, "asym", Y0)
    Y_ref, A = orc.matmul_ref(X_bits, packed, scales, zeros, 64, "asym")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        Xd = dev_bf16(X_bits)
        Y = torch.empty((3, 64), dtype=torch.bfloat16, device="cuda")
        q4.matmul_into(Xd, p, s, z, 64, "asym", Y)
    stream.synchronize()
    ok, usage = orc.check_matmul(host_bf16_to_f64(Y), Y_ref, A)
    assert ok, usage


@pytest.mark.parametrize("M,N,K,g", [(512, 8192, 256, 128), (520, 8100, 256, 32),
                                     (1024, 8192, 256, 128), (1000, 8000, 384, 64),
                                     (1088, 16384, 256, 128)])
def test_prefill_tile_choices(M, N, K, g):
    """The GEMM's tile choice on a 256-CU device: 256 x 256 tiles when they fill every compute
    unit (last shape), otherwise 128 x 128 tiles (the 128 x 256 tile would need twice as many
    tiles as units, which the 256 x 256 tile already covers at this CU count), full and with
    ragged M and N edges."""
    import torch
    from tests.gpu_util import log
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    large = -(-M // 256) * -(-N // 256)
    wide = -(-M // 128) * -(-N // 256)
    kind = "256x256" if large >= cus else ("128x256" if wide >= 2 * cus else "128x128")
    log(f"tile choice M={M} N={N} on {cus} CUs: {kind} tiles")
    rng = np.random.default_rng(M + N + K + g + 1)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full(X_bits, W_bits, g, mode, "prefill-tiles", ("auto",))
