"""Every entry point recorded into a HIP graph replays to the eager result, bit for bit.

Decode loops in serving replay captured graphs.  The library launches only kernels on the
caller's stream (no allocation, no host synchronisation, no memset nodes), so a captured
sequence must give exactly what the same calls give eagerly: the kernels are deterministic.
The graph here holds the 4-bit quantize, the matmul at decode (M = 1, 3) and prefill (M = 80)
sizes, the standalone dequantize, the 8-bit quantize and matmul, the AWQ search and GPTQ.  It is
replayed several times; between replays every output is overwritten and the same entry points run
eagerly on other inputs, and each replay is checked against the eager result.
"""
import numpy as np
import pytest

from synth import f64_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    from tests.gpu_util import require_gpu
    require_gpu()


def _inputs(seed, N=256, K=1024, g=128):
    import torch
    from tests.gpu_util import dev_bf16
    rng = np.random.default_rng(seed)
    W = dev_bf16(f64_to_bf16_bits(rng.normal(0, 0.05, (N, K))))
    X = {M: dev_bf16(f64_to_bf16_bits(rng.normal(0, 1, (M, K)))) for M in (1, 3, 80)}
    Xc = dev_bf16(f64_to_bf16_bits(rng.normal(0, 1, (128, K))))
    Yref = (Xc.float() @ W.float().t()).to(torch.bfloat16)
    return W, X, Xc, Yref


def _outputs(N=256, K=1024, g=128, M_awq=128, n_alpha=5):
    import torch
    import weight_only_int4_group_amd as q4
    d = torch.device("cuda:0")
    G = K // g
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=d)
    f16 = lambda *s: torch.empty(s, dtype=torch.float16, device=d)
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=d)
    return {
        "p": u8(N, K // 2), "s": f16(N, G), "z": u8(N, G),
        "Y1": bf(1, N), "Y3": bf(3, N), "Y80": bf(80, N), "deq": bf(N, K),
        "c8": u8(N, K), "s8": f16(N, G), "z8": u8(N, G), "Y8_1": bf(1, N), "Y8_80": bf(80, N),
        "awq_ws": u8(q4.awq_workspace_bytes(M_awq, N, K, g, n_alpha)),
        "awq_s": torch.empty(K, dtype=torch.float32, device=d), "awq_p": u8(N, K // 2),
        "awq_sc": f16(N, G), "awq_z": u8(N, G),
        "awq_err": torch.empty(n_alpha, dtype=torch.float64, device=d),
        "awq_best": torch.empty(1, dtype=torch.int32, device=d),
        "gq_ws": u8(q4.gptq_workspace_bytes(M_awq, N, K, g)), "gq_p": u8(N, K // 2),
        "gq_s": f16(N, G), "gq_z": u8(N, G), "gq_info": torch.empty(1, dtype=torch.int32, device=d),
    }


def _calls(inp, o, g=128, n_alpha=5):
    import weight_only_int4_group_amd as q4
    W, X, Xc, Yref = inp
    q4.quantize_rtn_into(W, g, "asym", o["p"], o["s"], o["z"])
    for M in (1, 3, 80):
        q4.matmul_into(X[M], o["p"], o["s"], o["z"], g, "asym", o[f"Y{M}"])
    q4.dequantize_into(o["p"], o["s"], o["z"], g, "asym", o["deq"])
    q4.quantize_rtn8_into(W, g, "sym", o["c8"], o["s8"], o["z8"])
    q4.matmul_w8_into(X[1], o["c8"], o["s8"], o["z8"], g, "sym", o["Y8_1"])
    q4.matmul_w8_into(X[80], o["c8"], o["s8"], o["z8"], g, "sym", o["Y8_80"])
    q4.awq_search_into(Xc, Yref, W, g, "asym", n_alpha, o["awq_ws"], o["awq_s"], o["awq_p"],
                       o["awq_sc"], o["awq_z"], o["awq_err"], o["awq_best"])
    q4.gptq_into(Xc, W, g, "sym", 0.01, o["gq_ws"], o["gq_p"], o["gq_s"], o["gq_z"], o["gq_info"])


def _snapshot(o):
    return {k: v.clone() for k, v in o.items() if not k.endswith("_ws")}


def test_graph_replays_match_eager():
    import torch
    from tests.gpu_util import log
    inp, other = _inputs(1), _inputs(2)
    o, o_other = _outputs(), _outputs()
    _calls(inp, o)
    torch.cuda.synchronize()
    eager = _snapshot(o)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _calls(inp, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _calls(inp, o)
    torch.cuda.synchronize()

    for rep in range(3):
        for k, v in o.items():
            if not k.endswith("_ws"):
                v.view(torch.uint8).fill_(0x5A + rep)
        _calls(other, o_other)       # eager work between replays, on the same kernels
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(o)
        bad = [k for k in eager if not torch.equal(got[k].view(torch.uint8), eager[k].view(torch.uint8))]
        log(f"graph replay {rep}: {len(eager) - len(bad)} of {len(eager)} outputs identical to eager")
        assert not bad, f"replay {rep}: outputs differ from the eager run: {bad}"
    assert int(eager["gq_info"].item()) == 0
    del graph
