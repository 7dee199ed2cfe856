"""q4_awq_search_static (the search in the library's static device scratch, for callers that
cannot allocate) against q4_awq_search on a caller's workspace: the same kernels on the same
inputs, so every output must be identical, bit for bit.  Two calls in a row, the second on a
smaller layer (the scratch keeps the first call's contents); then a layer larger than the
scratch is rejected before any launch.
"""
import numpy as np
import pytest

from synth import f64_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from tests.gpu_util import require_gpu
    require_gpu()


def _layer(N, K, M, seed):
    """Seeded bf16 W ~ N(0, 0.02), X ~ N(0, 1) with a few salient channels, Yref = X W^T (bf16)."""
    import torch
    from tests.gpu_util import dev_bf16
    rng = np.random.default_rng(seed)
    X = rng.normal(0, 1, (M, K))
    X[:, rng.choice(K, 8, replace=False)] *= 30.0
    W = rng.normal(0, 0.02, (N, K))
    Xd, Wd = dev_bf16(f64_to_bf16_bits(X)), dev_bf16(f64_to_bf16_bits(W))
    Yref = (Xd.float() @ Wd.float().T).to(torch.bfloat16)
    return Xd, Wd, Yref


def _outputs(N, K, g, n_alpha, dev):
    import torch
    return (torch.full((K,), float("nan"), dtype=torch.float32, device=dev),
            torch.full((N, K // 2), 0xAA, dtype=torch.uint8, device=dev),
            torch.full((N, K // g), float("nan"), dtype=torch.float16, device=dev),
            torch.full((N, K // g), 0xAA, dtype=torch.uint8, device=dev),
            torch.full((n_alpha,), float("nan"), dtype=torch.float64, device=dev),
            torch.full((1,), -1, dtype=torch.int32, device=dev))


def _check_pair(N, K, M, g, mode, n_alpha, seed):
    import torch
    import weight_only_int4_group_amd as q4
    from tests.gpu_util import log
    X, W, Yref = _layer(N, K, M, seed)
    ref = q4.awq_search(X, Yref, W, g, mode, n_alpha)
    out = _outputs(N, K, g, n_alpha, W.device)
    q4.awq_search_static_into(X, Yref, W, g, mode, n_alpha, *out)
    torch.cuda.synchronize()
    for name, a, b in zip(("s", "packed", "scales", "zeros", "errors", "best"), out, ref):
        a_h, b_h = a.cpu(), b.cpu()
        if a_h.dtype in (torch.float16, torch.float32, torch.float64):
            a_h = a_h.view({torch.float16: torch.int16, torch.float32: torch.int32, torch.float64: torch.int64}[a_h.dtype])
            b_h = b_h.view(a_h.dtype)
        assert torch.equal(a_h, b_h), f"static-scratch search: {name} differs (N={N} K={K} M={M} g={g} {mode})"
    log(f"awq_search_static N={N} K={K} M={M} g={g} {mode} n_alpha={n_alpha}: identical to the "
        f"workspace form (best {int(out[5].item())})")


def test_static_scratch_matches_workspace_form_twice_then_smaller():
    _check_pair(512, 2048, 64, 128, "asym", 11, seed=5)
    _check_pair(96, 512, 16, 64, "sym", 6, seed=6)        # second call: smaller, other mode


def test_static_scratch_rejects_a_layer_beyond_its_size():
    import torch
    import weight_only_int4_group_amd as q4
    N, K, M, g, n_alpha = 16384, 16384, 256, 128, 11
    assert q4.awq_workspace_bytes(M, N, K, g, n_alpha) > q4.awq_static_scratch_bytes()
    lib = q4.library()
    st = lib.q4_awq_search_static(None, M, None, None, N, K, g, 0, n_alpha, None, None, None, None, None,
                                  None, torch.cuda.current_stream().cuda_stream)
    assert st == -11 and "static buffer" in q4.status_string(st)
