"""GPU parity of the W8A16 path (8-bit group-wise RTN and its matmul) against the CPU oracle.

* q4_quantize_rtn8 is bit-exact against the oracle's 8-bit quantizer (codes, fp16 scales and
  zero-points), for every group-size path (power-of-two lane groups, any multiple of 32, g = K),
  both modes, special values, and the 70B MLP weight (all rows quantized on the GPU, a sample
  of row blocks compared).
* q4_matmul_w8 meets |Y - Y_ref| <= 8e-3 * sum_k |x w_hat| + 1e-6 per element for every kernel
  that can run the shape, on codes quantized by the oracle (never by the GPU): ragged shapes,
  M from 1 to 300 (decode GEMV and the general GEMM), ragged and large-tile shapes with M >= 512
  (the register-dequantising GEMM), on-grid weights against the exact product, special values,
  the 70B MLP shape at M = 1, 2, 4 and the prefill shape (sampled outputs).
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


def kernels_w8(M, K):
    """Every kernel that can run this shape (the rules stated in include/q4.h)."""
    ks = ["auto", "gemm"]
    if 1 <= M <= 4 and 2 * M * K + 4 * M * (K // 16) + 16 <= 160 * 1024:
        ks.append("gemv")
    return tuple(ks)


def _upload(codes, scales, zeros):
    import torch
    from tests.gpu_util import dev
    return dev(codes), dev(scales.view(np.uint16)).view(torch.float16), dev(zeros)


def _quant_gpu(W_bits, g, mode):
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import dev_bf16, host_u16
    c, s, z = q4.quantize_rtn8(dev_bf16(W_bits), g, mode)
    torch.cuda.synchronize()
    return c.cpu().numpy(), host_u16(s), z.cpu().numpy()


def _same(got, ref, label):
    for name, a, b in zip(("codes", "scales", "zeros"), got, (ref[0], ref[1].view(np.uint16), ref[2])):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)[:5]
            raise AssertionError(f"{label}: {name} differ at {bad.tolist()}")


# ------------------------------------------------------------------------------ quantize
@pytest.mark.parametrize("N,K,g", [(64, 256, 32), (33, 1024, 64), (17, 2048, 128), (8, 4096, 256),
                                   (5, 1536, 512), (19, 480, 96), (7, 960, 160), (4, 768, 384),
                                   (3, 8192, 8192), (1, 32, 32), (300, 640, 128)])
@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_quantize8_bitexact(N, K, g, mode):
    from tests.gpu_util import log
    rng = np.random.default_rng(N * 7 + K + g)
    W = rng.normal(0, 0.02, (N, K))
    W[0, : min(g, K)] *= 40.0                           # an outlier group
    W_bits = f64_to_bf16_bits(W)
    _same(_quant_gpu(W_bits, g, mode), orc.quantize8_rtn_ref(W_bits, g, mode), f"N={N} K={K} g={g} {mode}")
    log(f"quantize8 parity ok: N={N} K={K} g={g} {mode}")


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_quantize8_special_values(mode):
    rng = np.random.default_rng(5)
    N, K, g = 12, 256, 64
    W = rng.normal(0, 0.02, (N, K))
    W[0] = 0.0                                         # all-zero row: scale 1.0, codes 0
    W[1] = 0.37                                        # constant positive
    W[2] = -0.37                                       # constant negative
    W[3] = 1e-10                                       # scale underflows fp16 -> stored as 1.0
    W[4] = rng.normal(0, 1e30, K)                      # scale saturates at 65504
    W[5, ::2] = 3e38; W[5, 1::2] = -3e38               # range overflows fp32 in beta - alpha
    W[6] = np.abs(W[6])
    W[7] = -np.abs(W[7])
    W[8, :64] = 0.0; W[8, 0] = -1.0                    # one large negative among zeros: z = 255
    W[9] = np.round(rng.normal(0, 40, K)) * 2.0 ** -7  # on the code grid
    # ties: x / s exactly k + 1/2 for a power-of-two scale
    W[10] = (rng.integers(-120, 120, K) + 0.5) * 2.0 ** -10
    W[10, ::64] = 127 * 2.0 ** -10
    W[11] = rng.standard_normal(K) * np.exp2(rng.integers(-20, 20, K))
    W_bits = f64_to_bf16_bits(W)
    _same(_quant_gpu(W_bits, g, mode), orc.quantize8_rtn_ref(W_bits, g, mode), f"special {mode}")


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_quantize8_exhaustive_bf16_values(mode):
    """Every finite bf16 pattern, each next to the same group-range setters, so each value is
    quantized under several scales (the code decision is taken in fp32 on both sides)."""
    vals = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = orc.bf16_bits_to_f32(vals)
    vals = vals[np.isfinite(f) & (np.abs(f) < 1e30)]
    g = 32
    n = -(-len(vals) // 30)
    n += -n % 8                                        # groups: a multiple of 8 (rows of 256)
    body = np.resize(vals, n * 30).reshape(n, 30)      # 30 values per group
    rng = np.random.default_rng(9)
    setters = f64_to_bf16_bits(rng.choice([1.0, 3.5, 100.0, 1e-3, 7e4], (n, 1)) * np.array([[1.0, -1.0]]))
    W_bits = np.concatenate([setters, body], axis=1).reshape(-1, 8 * g)
    _same(_quant_gpu(W_bits, g, mode), orc.quantize8_rtn_ref(W_bits, g, mode), f"exhaustive {mode}")


@pytest.fixture(scope="module")
def layer70b_w8():
    cfg = CONFIGS[3]
    W_bits, X_bits = make_layer(cfg)
    return cfg, W_bits, X_bits, orc.quantize8_rtn_ref(W_bits, cfg.g, "sym")


def test_quantize8_70b_shape(layer70b_w8):
    """All 28672 x 8192 weights quantized on the GPU; rows 0-511, a middle block and the last
    512 rows compared bit for bit with the oracle's full quantization."""
    cfg, W_bits, _, ref = layer70b_w8
    got = _quant_gpu(W_bits, cfg.g, "sym")
    for lo in (0, cfg.N // 2 - 256, cfg.N - 512):
        sl = slice(lo, lo + 512)
        _same(tuple(a[sl] for a in got), tuple(b[sl] for b in ref), f"70b rows {lo}..")


# ------------------------------------------------------------------------------ matmul
def _gpu_mm8(X_bits, qw, g, mode, kernel="auto"):
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import dev_bf16, host_bf16_to_f64
    c, s, z = qw
    Y = q4.matmul_w8(dev_bf16(X_bits), c, s, z, g, mode, kernel)
    torch.cuda.synchronize()
    return host_bf16_to_f64(Y)


def _check_full8(X_bits, W_bits, g, mode, label, kernels, quant=None):
    from tests.gpu_util import log
    codes, scales, zeros = quant if quant is not None else orc.quantize8_rtn_ref(W_bits, g, mode)
    Y_ref, A = orc.matmul8_ref(X_bits, codes, scales, zeros, g, mode)
    qw = _upload(codes, scales, zeros)
    Y = None
    for kernel in kernels:
        Y = _gpu_mm8(X_bits, qw, g, mode, kernel)
        ok, usage = orc.check_matmul(Y, Y_ref, A)
        log(f"w8 matmul {label} kernel={kernel} M={X_bits.shape[0]} N={codes.shape[0]} K={X_bits.shape[1]} "
            f"g={g} {mode}: max tolerance usage {usage:.3e}")
        assert ok, f"{label} kernel={kernel}: tolerance exceeded (usage {usage})"
    return Y


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16, 17, 64, 129, 300])
@pytest.mark.parametrize("N,K,g", [(100, 96, 32), (37, 256, 64), (128, 4096, 128), (1, 32, 32),
                                   (50, 640, 128), (33, 1024, 256), (20, 8192, 8192), (64, 480, 96)])
def test_matmul_w8_ragged(M, N, K, g):
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full8(X_bits, W_bits, g, mode, "ragged", kernels_w8(M, K))


@pytest.mark.parametrize("log2_ratio", [12, 24, 31, 36, 60])
@pytest.mark.parametrize("N,K,g", [(256, 4096, 128), (80, 1024, 32)])
def test_matmul_w8_adversarial_dynamic_range(log2_ratio, N, K, g):
    """Small same-sign activations and, in every 128-weight block, one activation 2^log2_ratio
    larger that meets a zero weight (code equal to the zero point): the small ones carry all of
    Y, so none may be lost to the fp16 staging of X."""
    from tests.test_gpu_matmul import adversarial_layer
    for M in (1, 2, 4, 5):
        W_bits, X_bits = adversarial_layer(N, K, M, log2_ratio, seed=log2_ratio + M)
        for mode in ("asym", "sym"):
            _check_full8(X_bits, W_bits, g, mode, f"adversarial 2^{log2_ratio}", kernels_w8(M, K))


@pytest.mark.parametrize("M,K", [(1, 65536), (2, 28672), (4, 16384), (3, 16384)])
def test_matmul_w8_gemv_lds_limits(M, K):
    """The largest X the decode GEMV stages in LDS (2.25 M K bytes up to 160 KiB)."""
    rng = np.random.default_rng(M + K)
    N, g = 70, 128
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    assert "gemv" in kernels_w8(M, K)
    for mode in ("asym", "sym"):
        _check_full8(X_bits, W_bits, g, mode, "lds-limit", ("gemv",))


def test_matmul_w8_special_values():
    rng = np.random.default_rng(7)
    N, K, g = 48, 512, 128
    W = rng.normal(0, 0.02, (N, K))
    W[0] = 0.0                                   # all-zero row: Y must be exactly 0
    W[1, :128] = 0.0                             # one all-zero group
    W[2] = 0.5                                   # constant row
    W[3] = np.abs(W[3])
    W[4] = 1e-10                                 # scale underflow -> 1.0
    W[5, :] = 1e-4; W[5, ::128] = -1.0           # z = 255 with codes near z in every group
    W_bits = f64_to_bf16_bits(W)
    X = rng.normal(0, 1, (6, K))
    X[1] = 0.0                                   # all-zero activation row
    X[2, :] = 1e-20; X[2, ::7] = 1e20            # huge dynamic range within a 16-weight chunk
    X[3] = 1.0
    X[4, :] = 0.0; X[4, 5] = 1.0                 # one-hot
    X[5] = rng.normal(0, 1, K) * np.exp2(rng.integers(-60, 60, K))
    X_bits = f64_to_bf16_bits(X)
    for mode in ("asym", "sym"):
        for M in (1, 2, 4, 6):
            Y = _check_full8(X_bits[:M], W_bits, g, mode, "special", kernels_w8(M, K))
            assert np.all(Y[:, 0] == 0.0)


def test_matmul_w8_on_grid_weights_match_exact_product():
    """W = s (q - z) exactly (s a power of two, all 256 codes used): the quantizer reproduces W,
    so Y must meet the bound against X W^T itself."""
    rng = np.random.default_rng(21)
    N, K, g = 64, 1024, 128
    G = K // g
    z = rng.integers(0, 256, (N, G))
    q = rng.integers(0, 256, (N, G, g)); q[..., 0], q[..., 1] = 0, 255
    W = ((q - z[..., None]) * 2.0 ** -9).reshape(N, K)
    W_bits = f64_to_bf16_bits(W)
    assert np.array_equal(orc.bf16_bits_to_f32(W_bits).astype(np.float64), W)
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (20, K)))
    codes, scales, zeros = orc.quantize8_rtn_ref(W_bits, g, "asym")
    assert np.array_equal(orc.dequantize8_ref(codes, scales, zeros, g, "asym"), W)
    X = orc.bf16_bits_to_f32(X_bits).astype(np.float64)
    exact, A = X @ W.T, np.abs(X) @ np.abs(W).T
    qw = _upload(codes, scales, zeros)
    for M in (1, 2, 4, 7, 20):
        for kernel in kernels_w8(M, K):
            Y = _gpu_mm8(X_bits[:M], qw, g, "asym", kernel)
            assert np.all(np.abs(Y - exact[:M]) <= orc.tol_ref(A[:M])), (M, kernel)


def _check_sampled8(X_bits, quant, g, mode, label, kernel, n_samples=3000, seed=0):
    from tests.gpu_util import log
    codes, scales, zeros = quant
    Y = _gpu_mm8(X_bits, _upload(codes, scales, zeros), g, mode, kernel)
    M, N = Y.shape
    rng = np.random.default_rng(seed)
    mi = np.concatenate([rng.integers(0, M, n_samples), [0, M - 1, 0, M - 1]])
    ni = np.concatenate([rng.integers(0, N, n_samples), [0, 0, N - 1, N - 1]])
    rows = np.unique(ni)
    What = orc.dequantize8_ref(codes[rows], scales[rows], zeros[rows], g, mode)
    pos = np.searchsorted(rows, ni)
    X = orc.bf16_bits_to_f32(X_bits).astype(np.float64)
    Y_ref = np.einsum("ij,ij->i", X[mi], What[pos])
    A = np.einsum("ij,ij->i", np.abs(X[mi]), np.abs(What[pos]))
    ok, usage = orc.check_matmul(Y[mi, ni], Y_ref, A)
    log(f"w8 matmul (sampled) {label} kernel={kernel} M={M} N={N} g={g} {mode}: max tolerance usage {usage:.3e}")
    assert ok, f"{label}: tolerance exceeded (usage {usage})"


@pytest.mark.parametrize("M", [1, 2, 4])
def test_matmul_w8_70b_mlp_decode(layer70b_w8, M):
    cfg, _, X_bits, quant = layer70b_w8
    for kernel in kernels_w8(M, cfg.K):
        _check_sampled8(X_bits[:M], quant, cfg.g, "sym", cfg.name, kernel)


def test_matmul_w8_prefill():
    cfg = CONFIGS[4]
    W_bits, X_bits = make_layer(cfg)
    quant = orc.quantize8_rtn_ref(W_bits, cfg.g, "asym")
    _check_sampled8(X_bits, quant, cfg.g, "asym", cfg.name, "auto", n_samples=4096)


@pytest.mark.parametrize("M,N,K,g", [(512, 64, 128, 128), (513, 300, 256, 32), (640, 256, 384, 128),
                                     (1000, 520, 512, 64), (700, 1030, 1024, 256), (777, 136, 640, 128)])
def test_matmul_w8_prefill_ragged(M, N, K, g):
    """Large-M shapes on the register-dequantising GEMM with 8-bit codes: ragged M and N tiles,
    odd step counts, every power-of-two g."""
    rng = np.random.default_rng(M + 3 * N + 7 * K + g)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full8(X_bits, W_bits, g, mode, "prefill-ragged", ("auto", "gemm"))


@pytest.mark.parametrize("M,N,K,g", [(589, 22000, 384, 128), (512, 32768, 256, 32), (1024, 16384, 512, 256),
                                     (600, 21800, 640, 64)])
def test_matmul_w8_prefill_large_tiles(M, N, K, g):
    """Shapes with enough 256 x 256 tiles to fill the device, so the 256-row tile runs with
    8-bit codes: ragged M and N, every g, both modes."""
    rng = np.random.default_rng(M + N + K + g)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full8(X_bits, W_bits, g, mode, "prefill-large", ("auto",))


def test_matmul_w8_m0_nondefault_stream_and_determinism():
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import dev_bf16
    rng = np.random.default_rng(3)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (96, 512)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (4, 512)))
    c, s, z = _upload(*orc.quantize8_rtn_ref(W_bits, 64, "asym"))
    Y0 = torch.full((0, 96), 1.0, dtype=torch.bfloat16, device="cuda")
    q4.matmul_w8_into(dev_bf16(X_bits[:0]), c, s, z, 64, "asym", Y0)
    X = dev_bf16(X_bits)
    st = torch.cuda.Stream()
    for kernel in kernels_w8(4, 512):
        ref = q4.matmul_w8(X, c, s, z, 64, "asym", kernel)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            Y = torch.empty((4, 96), dtype=torch.bfloat16, device="cuda")
            q4.matmul_w8_into(X, c, s, z, 64, "asym", Y, kernel)
        st.synchronize()
        assert torch.equal(Y, ref), kernel
