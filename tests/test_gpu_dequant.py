"""GPU standalone dequantisation parity: every output element must be bit-identical to the
oracle's exact x_hat = scale * (q - z) rounded once to bf16 / fp16 (round half to even).

Inputs are either quantized by the oracle on the host from seeded bf16 weights, or raw
seeded codes, scales and zero-points (to reach fp16 subnormal scales and fp16 overflow).
Each call writes into a buffer with a guard region behind it, which must stay untouched.
"""
import numpy as np
import pytest

from oracle import q4_oracle as orc
from synth import CONFIGS, f64_to_bf16_bits, make_layer

pytestmark = pytest.mark.gpu

GUARD = 4096          # elements after the output that the call must not write


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from tests.gpu_util import require_gpu
    require_gpu()


def _gpu_dequant(packed, scales, zeros, g, mode, out):
    """Run q4_dequantize into a guarded buffer; returns the output's bit patterns (uint16)."""
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import dev
    N, K = packed.shape[0], packed.shape[1] * 2
    dtype = torch.bfloat16 if out == "bf16" else torch.float16
    buf = torch.full((N * K + GUARD,), -7.0, dtype=dtype, device="cuda")
    p = dev(packed)
    s = dev(np.asarray(scales, dtype=np.float16).view(np.uint16)).view(torch.float16)
    z = None if (mode == "sym" and zeros is None) else dev(zeros)
    q4.dequantize_into(p, s, z, g, mode, buf[:N * K].view(N, K))
    torch.cuda.synchronize()
    host = buf.cpu().view(torch.int16).numpy().view(np.uint16)
    sentinel = torch.tensor([-7.0], dtype=dtype).view(torch.int16).numpy().view(np.uint16)[0]
    assert np.all(host[N * K:] == sentinel), "dequantize wrote past the end of its output"
    return host[:N * K].reshape(N, K)


def _check(packed, scales, zeros, g, mode, label, outs=("bf16", "f16")):
    from tests.gpu_util import log
    for out in outs:
        got = _gpu_dequant(packed, scales, zeros, g, mode, out)
        want = orc.dequantize_rounded_ref(packed, scales, zeros, g, mode, out)
        want = want if out == "bf16" else want.view(np.uint16)
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)[:5]
            raise AssertionError(f"{label} g={g} {mode} {out}: differs at {bad.tolist()}: "
                                 f"gpu {[hex(got[tuple(i)]) for i in bad]} "
                                 f"oracle {[hex(want[tuple(i)]) for i in bad]}")
        log(f"dequantize parity ok: {label} N={packed.shape[0]} K={packed.shape[1] * 2} g={g} "
            f"{mode} {out}")


def _quantized(N, K, g, mode, seed):
    rng = np.random.default_rng(seed)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (N, K)))
    return orc.quantize_rtn_ref(W_bits, g, mode)


# Power-of-two and other group sizes (g / 8 dwords per group: 4 .. 3584), ragged chunk tails
# (N K / 8 not a multiple of 256), one group per row (g = K).
@pytest.mark.parametrize("N,K,g", [(1, 32, 32), (3, 96, 32), (7, 640, 128), (33, 1024, 256),
                                   (5, 480, 160), (9, 384, 96), (17, 8192, 8192),
                                   (2, 28672, 28672), (129, 2048, 64), (61, 1536, 512)])
@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_dequantize_shapes(N, K, g, mode):
    packed, scales, zeros = _quantized(N, K, g, mode, N * 7 + K + g)
    _check(packed, scales, zeros, g, mode, "shapes")


@pytest.mark.parametrize("N,K,g", [(4608, 4096, 128), (6000, 8640, 160), (4608, 7200, 96)])
def test_dequantize_persistent_strides(N, K, g):
    """More chunks than the persistent grid has waves on a 256-CU device, so waves take
    several chunks and carry the group position from one to the next (g / 8 = 16, 20, 12)."""
    for mode in ("asym", "sym"):
        packed, scales, zeros = _quantized(N, K, g, mode, N + K + g)
        _check(packed, scales, zeros, g, mode, "persistent", outs=("bf16",) if mode == "sym" else ("bf16", "f16"))


def test_dequantize_workload_layer():
    """The 8192 x 8192 layer of the prefill workload, quantized at its group size."""
    cfg = CONFIGS[4]
    W_bits, _ = make_layer(cfg)
    packed, scales, zeros = orc.quantize_rtn_ref(W_bits, cfg.g, cfg.mode)
    _check(packed, scales, zeros, cfg.g, cfg.mode, cfg.name, outs=("bf16",))


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_dequantize_raw_codes_extreme_scales(mode):
    """Arbitrary codes and zero-points with fp16 scales from subnormal to 65504: bf16 is
    exact or rounded, fp16 results beyond its range become inf."""
    rng = np.random.default_rng(17 if mode == "asym" else 18)
    N, K, g = 37, 1280, 64
    packed = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    expo = rng.uniform(-24, 15.9, (N, K // g))
    scales = np.exp2(expo).astype(np.float16)
    scales[0, :4] = np.array([2.0 ** -24, 3 * 2.0 ** -24, 65504.0, 4097.0], dtype=np.float16)
    zeros = rng.integers(0, 16, (N, K // g)).astype(np.uint8)
    _check(packed, scales, zeros, g, mode, "raw")


def test_dequantize_sym_accepts_null_zeros():
    packed, scales, _ = _quantized(8, 256, 32, "sym", 3)
    _check(packed, scales, None, 32, "sym", "sym-null-zeros")
