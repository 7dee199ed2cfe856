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


def decode_fits(M, N, K, g, mode="asym"):
    """Whether Q4_KERNEL_DECODE runs this shape (the rule stated in include/q4.h)."""
    if not (1 <= M <= 16 and g in (32, 64, 128)) or N * (K // 2) >= 2 ** 32:
        return False
    P = 4 if M <= 4 else (2 if M <= 8 else 1)
    S = 8 if (g == 32 and P >= 2) or (g == 64 and P == 4) else 16
    if P == 4 and K % 1024 == 0 and K // 1024 <= 8:
        S = 8
    while S > 4 and P * (S // 2) >= 16 and (K % (32 * P * S) != 0 or K // (32 * P * S) < 4):
        S //= 2
    if P == 1 and g >= 64 and K // 512 > 8 and K % 1024 == 0:
        S = 32
    KR = 32 * P * S
    if K % KR != 0 or KR < 512 or KR // g < 4 or K // KR > 8:
        return False
    NG = KR // g
    stage = 16 * (KR // 2) + 256 * ((8 * NG + 63) // 64) + 256 * ((4 * NG + 63) // 64)
    return 2 * (K // KR) * stage + 2 * (K // KR) * 1024 <= 160 * 1024


def decode_rows_fit(M, N, K, g):
    """Whether Q4_KERNEL_DECODE runs M rows: launches of 16 rows, the last M mod 16, each fitting."""
    if M <= 16:
        return decode_fits(M, N, K, g)
    return decode_fits(16, N, K, g) and (M % 16 == 0 or decode_fits(M % 16, N, K, g))


def kernels_for(M, N, K, g):
    """Every kernel that can run this shape (mirrors the rules stated in include/q4.h)."""
    ks = ["auto", "gemm"]
    if (M == 1 and K <= 16384) or (M == 2 and K <= 4096):
        ks.append("gemv")
    if decode_rows_fit(M, N, K, g):
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


@pytest.fixture(scope="module")
def layer70b():
    cfg = CONFIGS[3]
    W_bits, X_bits = make_layer(cfg)
    return cfg, X_bits, orc.quantize_rtn_ref(W_bits, cfg.g, cfg.mode)


def _check_every_element(Y, X_bits, qw_host, g, mode, label, kernel, row_block=4096):
    """Every element of a full-size Y against the oracle, W rows in blocks (bounded memory)."""
    from tests.gpu_util import log
    packed, scales, zeros = qw_host
    worst = 0.0
    for r0 in range(0, packed.shape[0], row_block):
        r1 = min(r0 + row_block, packed.shape[0])
        Y_ref, A = orc.matmul_ref(X_bits, packed[r0:r1], scales[r0:r1], zeros[r0:r1], g, mode)
        ok, usage = orc.check_matmul(Y[:, r0:r1], Y_ref, A)
        worst = max(worst, usage)
        assert ok, f"{label} kernel={kernel} rows {r0}..{r1}: tolerance exceeded (usage {usage})"
    log(f"matmul parity (every element) {label} kernel={kernel} M={Y.shape[0]} N={Y.shape[1]} g={g} "
        f"{mode}: max tolerance usage {worst:.3e}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_70b_mlp_decode(layer70b, M):
    """The 70B-shaped layer at M = 1, 4, 8: every element of Y, for every kernel that runs it."""
    cfg, X_bits, qw = layer70b
    for kernel in kernels_for(M, cfg.N, cfg.K, cfg.g):
        Y = _gpu_matmul(X_bits[:M], _upload(*qw), cfg.g, cfg.mode, kernel)
        _check_every_element(Y, X_bits[:M], qw, cfg.g, cfg.mode, cfg.name, kernel)


def test_70b_mlp_decode_m16(layer70b):
    """The 70B-shaped layer at M = 16 (X drawn by the same recipe with 16 rows): every element
    of Y, for every kernel that runs it (the 32-slice decode among them)."""
    import dataclasses
    cfg, _, qw = layer70b
    _, X16 = make_layer(dataclasses.replace(cfg, M_max=16))
    ks = kernels_for(16, cfg.N, cfg.K, cfg.g)
    assert "decode" in ks
    for kernel in ks:
        Y = _gpu_matmul(X16, _upload(*qw), cfg.g, cfg.mode, kernel)
        _check_every_element(Y, X16, qw, cfg.g, cfg.mode, cfg.name + " M=16", kernel)


@pytest.fixture(scope="module")
def prefill_runs():
    """The prefill workload's Y (bench launch configuration: auto kernel) for g = 128 and 32."""
    cfg = CONFIGS[4]
    W_bits, X_bits = make_layer(cfg)
    out = {}
    for g in (128, 32):
        qw = orc.quantize_rtn_ref(W_bits, g, cfg.mode)
        out[g] = (qw, _gpu_matmul(X_bits, _upload(*qw), g, cfg.mode))
    return cfg, X_bits, out


@pytest.mark.parametrize("g", [128, 32])
@pytest.mark.parametrize("block", [0, 1, 2, 3])
def test_prefill(prefill_runs, g, block):
    """The prefill workload (M = 2048, 8192 x 8192), every element of Y: one quarter of the W
    rows per test."""
    cfg, X_bits, out = prefill_runs
    (packed, scales, zeros), Y = out[g]
    q = packed.shape[0] // 4
    r0, r1 = block * q, (block + 1) * q
    _check_every_element(Y[:, r0:r1], X_bits, (packed[r0:r1], scales[r0:r1], zeros[r0:r1]), g, cfg.mode,
                         f"{cfg.name} rows {r0}..{r1}", "auto", row_block=1024)


def adversarial_layer(N, K, M, log2_ratio, seed=0):
    """Activations of one sign and small magnitude, and in every 128-weight block one activation
    2^log2_ratio times larger that meets a zero weight (its code equals the zero point, so it
    adds nothing to Y or to the tolerance's sum |x x_hat|): a kernel that scales X per block
    into fp16 would lose the small activations, which carry all of Y."""
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.02, (N, K))
    big = np.arange(5, K, 128)
    W[:, big] = 0.0
    X = np.abs(rng.normal(0, 1e-3, (M, K))) + 1e-4
    X[:, big] = 1e-3 * 2.0 ** log2_ratio
    return f64_to_bf16_bits(W), f64_to_bf16_bits(X)


@pytest.mark.parametrize("log2_ratio", [12, 20, 24, 28, 36, 60])
@pytest.mark.parametrize("N,K,g", [(256, 4096, 128), (96, 1024, 32), (80, 2048, 64)])
def test_adversarial_dynamic_range(log2_ratio, N, K, g):
    for M in (1, 2, 4, 8, 16):
        W_bits, X_bits = adversarial_layer(N, K, M, log2_ratio, seed=log2_ratio + M)
        for mode in ("asym", "sym"):
            _check_full(X_bits, W_bits, g, mode, f"adversarial 2^{log2_ratio}", kernels_for(M, N, K, g))


@pytest.mark.parametrize("M,N,K,g", [(1, 33000, 1024, 128), (2, 33001, 1024, 64), (1, 17003, 8192, 128),
                                     (1, 17000, 6144, 128), (2, 33001, 4096, 128), (1, 33000, 1536, 512)])
def test_gemv_many_rows_per_wave(M, N, K, g):
    """GEMV shapes with at least four rows per wave on a 256-CU device, where each wave copies its
    contiguous rows' scales and zero-points into LDS once (4 | K / g; K / g = 3 keeps the per-row
    loads): every element of Y, ragged row counts, both modes."""
    rng = np.random.default_rng(N + K + g + M)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        qw = orc.quantize_rtn_ref(W_bits, g, mode)
        Y = _gpu_matmul(X_bits, _upload(*qw), g, mode, "gemv")
        _check_every_element(Y, X_bits, qw, g, mode, "gemv-many-rows", "gemv")


@pytest.mark.parametrize("M", [1, 2])
def test_gemv_many_rows_per_wave_exact_path(M):
    """X whose fp16 staging would lose bits (the exact fp32 path) on a many-rows-per-wave shape."""
    N, K, g = 33000, 1024, 128
    W_bits, X_bits = adversarial_layer(N, K, M, 36, seed=5 + M)
    for mode in ("asym", "sym"):
        qw = orc.quantize_rtn_ref(W_bits, g, mode)
        Y = _gpu_matmul(X_bits, _upload(*qw), g, mode, "gemv")
        _check_every_element(Y, X_bits, qw, g, mode, "gemv-many-rows-exact", "gemv")


@pytest.mark.parametrize("M,N,K,g", [(4, 8200, 4096, 64), (8, 8195, 2048, 32), (16, 8300, 4096, 128),
                                     (3, 8209, 8192, 128), (12, 8250, 1024, 64), (6, 9000, 8192, 128),
                                     (1, 8192, 512, 32), (4, 8200, 8192, 64)])
def test_decode_many_row_blocks(M, N, K, g):
    """Matrix-core decode on shapes with at least two 16-row blocks per workgroup on a 256-CU
    device, where the workgroup copies each row block's scales and zero-points into LDS slots
    shared by its waves (K = 8192 at g = 64 does not fit them and keeps the per-wave copies):
    every element of Y, ragged N, both modes."""
    assert decode_fits(M, N, K, g)
    rng = np.random.default_rng(N + K + g + M)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        qw = orc.quantize_rtn_ref(W_bits, g, mode)
        Y = _gpu_matmul(X_bits, _upload(*qw), g, mode, "decode")
        _check_every_element(Y, X_bits, qw, g, mode, "decode-many-blocks", "decode")


@pytest.mark.parametrize("M", [2, 5, 16])
def test_decode_many_row_blocks_exact_path(M):
    """X whose fp16 staging would lose bits (the bf16 exact path) with shared scale slots."""
    N, K, g = 8300, 2048, 128
    W_bits, X_bits = adversarial_layer(N, K, M, 36, seed=11 + M)
    for mode in ("asym", "sym"):
        qw = orc.quantize_rtn_ref(W_bits, g, mode)
        Y = _gpu_matmul(X_bits, _upload(*qw), g, mode, "decode")
        _check_every_element(Y, X_bits, qw, g, mode, "decode-many-blocks-exact", "decode")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8, 9, 12, 16])
@pytest.mark.parametrize("N,K,g", [(100, 1536, 64), (300, 2048, 128), (33, 4096, 32), (129, 8192, 64),
                                   (50, 3072, 128), (17, 512, 32), (257, 4096, 128), (70, 6144, 128)])
def test_decode_shapes(M, N, K, g):
    """Shapes the matrix-core decode kernel takes (K a multiple of 512, ragged N), every kernel."""
    rng = np.random.default_rng(M * 17 + N + K + g)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full(X_bits, W_bits, g, mode, "decode-shapes", kernels_for(M, N, K, g))


@pytest.mark.parametrize("M", [17, 20, 32, 33, 48, 64, 95])
@pytest.mark.parametrize("N,K,g", [(300, 2048, 128), (4096, 4096, 128), (129, 8192, 64), (70, 4096, 32)])
def test_decode_in_row_chunks(M, N, K, g):
    """M > 16 through the decode kernel in 16-row launches (and the choice auto makes), every
    element against the oracle; the last launch takes M mod 16 rows."""
    assert decode_rows_fit(M, N, K, g)
    rng = np.random.default_rng(M * 31 + N + K + g)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    X_bits = f64_to_bf16_bits(rng.normal(0, 1, (M, K)))
    for mode in ("asym", "sym"):
        _check_full(X_bits, W_bits, g, mode, "decode-row-chunks", kernels_for(M, N, K, g))


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
