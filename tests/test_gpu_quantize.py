"""GPU quantize parity: packed codes, fp16 scales and zero-points must be bit-identical to
the CPU oracle, on the workload shapes and on edge-case groups."""
import numpy as np
import pytest

from oracle import q4_oracle as orc
from synth import CONFIGS, f64_to_bf16_bits, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from tests.gpu_util import require_gpu
    require_gpu()


def _gpu_quant(W_bits, g, mode):
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import dev_bf16, host_u16
    p, s, z = q4.quantize_rtn(dev_bf16(W_bits), g, mode)
    torch.cuda.synchronize()
    return p.cpu().numpy(), host_u16(s), z.cpu().numpy()


def _assert_same(W_bits, g, mode, rows=None, label=""):
    from tests.gpu_util import log
    gp, gs, gz = _gpu_quant(W_bits, g, mode)
    ref_in = W_bits if rows is None else W_bits[rows]
    rp, rs, rz = orc.quantize_rtn_ref(ref_in, g, mode)
    if rows is not None:
        gp, gs, gz = gp[rows], gs[rows], gz[rows]
    rs = rs.view(np.uint16)
    for name, a, b in (("packed", gp, rp), ("scales", gs, rs), ("zeros", gz, rz)):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)[:5]
            raise AssertionError(f"{label} g={g} {mode}: {name} differs at {bad.tolist()}: "
                                 f"gpu {[a[tuple(i)] for i in bad]} oracle {[b[tuple(i)] for i in bad]}")
    log(f"quantize parity ok: {label} shape={W_bits.shape} g={g} {mode}")


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_configs_small_full(idx):
    cfg = CONFIGS[idx]
    W_bits, _ = make_layer(cfg, M=1)
    _assert_same(W_bits, cfg.g, cfg.mode, label=cfg.name)
    other = "sym" if cfg.mode == "asym" else "asym"
    _assert_same(W_bits, cfg.g, other, label=cfg.name + " (other mode)")


@pytest.mark.parametrize("idx,g", [(3, 128), (4, 128), (4, 32)])
def test_configs_full_size_every_row(idx, g):
    """The 70B-shaped and prefill weights at full size: every row bit for bit."""
    cfg = CONFIGS[idx]
    W_bits, _ = make_layer(cfg, M=1)
    _assert_same(W_bits, g, cfg.mode, label=cfg.name + " (every row)")


def _edge_rows(K, g, rng):
    """Rows made of special groups; K % g == 0."""
    G = K // g
    kinds = []
    for j in range(G):
        kind = j % 12
        if kind == 0:
            v = np.zeros(g)
        elif kind == 1:
            v = np.full(g, 0.37)
        elif kind == 2:
            v = np.full(g, -5.5)
        elif kind == 3:
            v = np.abs(rng.normal(0, 1, g)) + 0.1
        elif kind == 4:
            v = -np.abs(rng.normal(0, 1, g)) - 0.1
        elif kind == 5:
            v = rng.normal(0, 1e-39, g)                       # bf16 subnormals
        elif kind == 6:
            v = rng.normal(0, 1e-10, g)                       # fp16 scale underflows to 0
        elif kind == 7:
            v = rng.normal(0, 1e37, g); v[0] = 3.0e38         # scale saturates at 65504
        elif kind == 8:                                       # exact ties at odd zero-point
            z = int(rng.integers(0, 16)) | 1
            e = int(rng.integers(-12, 4))
            idx = rng.integers(0, 30, g) / 2.0 - z
            idx[0], idx[1] = -z, 15 - z
            v = np.clip(idx, -z, 15 - z) * 2.0 ** e
        elif kind == 9:                                       # ties in symmetric grid
            e = int(rng.integers(-12, 4))
            v = (rng.integers(-15, 16, g) / 2.0) * 2.0 ** e
            v[0] = 7 * 2.0 ** e
        elif kind == 10:
            v = np.zeros(g); v[int(rng.integers(0, g))] = rng.normal(0, 3)
        else:
            v = rng.normal(0, 0.02, g) * np.where(rng.random(g) < 0.05, 50.0, 1.0)
        kinds.append(v)
    return np.concatenate(kinds)


@pytest.mark.parametrize("g,K", [(32, 384), (64, 768), (128, 1536), (256, 3072), (512, 6144),
                                 (96, 1152), (160, 1920), (1024, 12288), (384, 384)])
@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_edge_groups(g, K, mode):
    rng = np.random.default_rng(g * 7 + K)
    rows = [_edge_rows(K, g, rng) for _ in range(5)]
    rows.append(rng.normal(0, 0.02, K))
    W_bits = f64_to_bf16_bits(np.stack(rows))
    _assert_same(W_bits, g, mode, label="edge")


@pytest.mark.parametrize("N,K,g", [(1, 32, 32), (3, 96, 32), (7, 288, 96), (5, 64, 64),
                                   (33, 4096, 4096), (257, 160, 32), (1000, 256, 128)])
@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_ragged_shapes(N, K, g, mode):
    rng = np.random.default_rng(N * 1000 + K)
    W_bits = f64_to_bf16_bits(rng.normal(0, 0.05, (N, K)))
    _assert_same(W_bits, g, mode, label="ragged")


def test_many_random_matrices():
    rng = np.random.default_rng(99)
    for t in range(20):
        N = int(rng.integers(1, 80))
        g = int(rng.choice([32, 64, 128]))
        K = g * int(rng.integers(1, 8))
        scale = float(10.0 ** rng.uniform(-6, 4))
        W_bits = f64_to_bf16_bits(rng.standard_t(3, (N, K)) * scale)
        _assert_same(W_bits, g, "asym" if t % 2 else "sym", label=f"random{t}")
