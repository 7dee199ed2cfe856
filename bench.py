#!/usr/bin/env python3
"""Benchmark of the W4A16 hot path on one MI355X.

One step is one pass of the whole path over synthetic inputs resident in HBM:
  1. quantize  -- group-wise INT4 RTN of the 70B-shaped MLP weight W[28672, 8192] (asym, g=128)
  2. decode    -- W4A16 GEMV, M = 1, through L layers of that shape, each with its own quantized
                  weight copy: 80 by default, the layer count of a 70B Llama decoder, so one
                  step is one token's pass through every layer's MLP up-projection (9.9 GB of
                  weights; the 256 MB Infinity Cache cannot serve them)
  3. prefill   -- W4A16 GEMM, M = 2048, W[8192, 8192] (asym, g=128 and g=32), through the same
                  L layers, each with its own quantized weight copy
The headline value is the decode GEMV's HBM throughput: algorithmic bytes (packed codes +
fp16 scales + uint8 zeros + X + Y) per launch / measured launch time, HIP events on the
launch stream.  The K timed passes run phase-major (all K quantizes, then the K x L decode
GEMVs, then the K x L prefill GEMMs of each group size), each phase between one pair of events.  The CPU-baseline leg times the oracle on a bounded sample and asserts parity of
sampled GPU outputs against it before timing (both skipped with --no-cpu-baseline).
Also reported: the W8A16 path (8-bit codes), the AWQ-style scaling search, and practical
ceilings (a plain streaming read, a device copy, the vendor bf16 GEMM) as context.

  python bench.py [--steps K] [--warmup W] [--gpus 1]
  python bench.py --summarize-counters FETCH_DIR WRITE_DIR   (writes the traffic summary)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV HBM GB/s (% of peak) at M=1; GEMM TFLOP/s at M=2048"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 vector
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_70b_mlp_m1_traffic.md")
GEMV_SRC = os.path.join(ROOT, "weight_only_int4_group_amd", "csrc", "gemv.hip")


def note(msg):
    """Progress of the run on stderr (the JSON result alone goes to stdout)."""
    print(f"bench: {msg} ({time.perf_counter() - _T0:.1f} s)", file=sys.stderr, flush=True)


_T0 = time.perf_counter()


def weight_bytes(N, K, g, mode):
    G = K // g
    return N * K // 2 + 2 * N * G + (N * G if mode == "asym" else 0)


def matmul_bytes(M, N, K, g, mode):
    return weight_bytes(N, K, g, mode) + 2 * M * K + 2 * M * N


def quantize_bytes(N, K, g):
    return 2 * N * K + N * K // 2 + 3 * N * (K // g)


def src_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic():
    """Traffic per GEMV launch from the committed counter summary, if it matches the source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    try:
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        d = json.loads(blob)
    except (IndexError, ValueError):
        return None
    if d.get("gemv_src_sha") != src_sha(GEMV_SRC):
        return None
    return d.get("traffic_bytes_per_launch")


def warm_up(torch, fn, seconds=0.025, batch=50):
    """Untimed launches fn(0), fn(1), ... until `seconds` of wall time have passed (synchronising
    every `batch` launches).  After a pause or a change of work the first 10-20 ms of launches run
    slower while the clocks settle; every measurement below starts from that settled state."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(batch):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return i


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=80,
                   help="decoder layers per step, each with its own quantized weight copy")
    p.add_argument("--no-check", action="store_true",
                   help="skip the parity assertion of the CPU-baseline leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-context", action="store_true",
                   help="skip the practical-ceiling measurements reported as context")
    p.add_argument("--no-awq", action="store_true",
                   help="skip the AWQ-style scaling search measurement")
    p.add_argument("--no-gptq", action="store_true",
                   help="skip the GPTQ measurement")
    p.add_argument("--no-w8", action="store_true",
                   help="skip the W8A16 (8-bit codes) measurements")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also launch one plain 512 MiB device copy (counter calibration)")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="per-kernel duration statistics of a rocprofv3 --kernel-trace csv run")
    return p.parse_args(argv)


# --------------------------------------------------------------------------- context
def measure_context(torch, q4, sets, X5, W5, w5, reps=10):
    """Practical ceilings on this GPU, measured after the timed steps and reported beside the
    kernels (not targets):
      * a plain streaming read of the decode weight bytes (libq4_bench.so, eight 16-byte loads
        in flight per lane, rotating over the weight copies as the GEMV does; the best of a few
        grid sizes), and torch's device copy of the same bytes (read + write);
      * the vendor bf16 GEMM (torch.matmul, hipBLASLt) on the prefill shape with unquantized
        bf16 weights;
      * the two-step alternative to the fused prefill GEMM: q4_dequantize of the INT4 weights
        to bf16, then the vendor GEMM."""
    import ctypes
    from weight_only_int4_group_amd.build import BENCH_LIB

    def timed(fn, n):
        warm_up(torch, fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    res = {}
    codes = [s[0] for s in sets]
    read_bytes = codes[0].numel()
    if os.path.exists(BENCH_LIB):
        lib = ctypes.CDLL(BENCH_LIB)
        lib.q4b_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
        lib.q4b_stream_read.restype = ctypes.c_int
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        sink = torch.empty(cus * 64 * 4, dtype=torch.int32, device=codes[0].device)
        stream = torch.cuda.current_stream().cuda_stream
        best = None
        for per_cu in (4, 8, 16, 32):
            blocks = cus * per_cu
            run = lambda i: lib.q4b_stream_read(codes[i % len(codes)].data_ptr(), read_bytes,
                                                sink.data_ptr(), blocks, stream)
            ms = timed(run, reps * len(codes))
            if best is None or ms < best[0]:
                best = (ms, blocks)
        res["stream_read"] = {"GB/s": round(read_bytes / (best[0] * 1e-3) / 1e9, 1), "bytes": read_bytes,
                              "us": round(best[0] * 1e3, 2), "blocks": best[1],
                              "how": "libq4_bench stream_read over one decode weight's packed codes, "
                                     "rotating over the copies; best of 4, 8, 16, 32 blocks per CU"}
    dst = torch.empty_like(codes[0])
    copy_ms = timed(lambda i: dst.copy_(codes[i % len(codes)]), reps * len(codes))
    res["device_copy"] = {"GB/s": round(2 * read_bytes / (copy_ms * 1e-3) / 1e9, 1),
                          "how": "torch copy_ of one decode weight's packed codes (read + write bytes)"}
    flops = 2.0 * X5.shape[0] * W5.shape[0] * X5.shape[1]
    mm_ms = timed(lambda i: torch.matmul(X5, W5.t()), reps)
    res["vendor_bf16_gemm"] = {"TFLOP/s": round(flops / (mm_ms * 1e-3) / 1e12, 1), "ms": round(mm_ms, 4),
                               "how": "torch.matmul (hipBLASLt) X[2048,8192] @ W[8192,8192]^T in bf16, unquantized W"}
    Wd = torch.empty_like(W5)
    p5, s5, z5 = w5[128]
    deq_ms = timed(lambda i: q4.dequantize_into(p5, s5, z5, 128, "asym", Wd), reps)
    two_ms = timed(lambda i: (q4.dequantize_into(p5, s5, z5, 128, "asym", Wd),
                              torch.matmul(X5, Wd.t())), reps)
    deq_bytes = p5.numel() + s5.numel() * 2 + z5.numel() + Wd.numel() * 2
    res["dequantize_then_vendor_gemm"] = {
        "ms": round(two_ms, 4), "TFLOP/s": round(flops / (two_ms * 1e-3) / 1e12, 1),
        "dequantize_ms": round(deq_ms, 4),
        "dequantize_GB/s": round(deq_bytes / (deq_ms * 1e-3) / 1e9, 1),
        "how": "q4_dequantize of the g=128 INT4 weights to bf16 [8192,8192], then torch.matmul"}
    return res


# --------------------------------------------------------------------------- AWQ-style scaling
def measure_awq(torch, q4, W5, X5, W5_bits, X5_bits, calib=512, g=128, n_alpha=11, reps=3,
                with_oracle=True, oracle_rows=512, oracle_calib=64):
    """AWQ-style scaling search on the prefill layer W[8192, 8192]: `calib` calibration rows of
    its activations, the unquantized layer output on them as the reference (torch.matmul, an
    input of the search, not timed), n_alpha grid points, g=128 asym.  Times q4_awq_search
    (HIP events on the launch stream) and, alone, the scaled RTN quantization it runs per alpha
    (HBM roofline).  The oracle's awq_search_ref is timed beside it on a bounded sample
    (`oracle_rows` rows of W, `oracle_calib` calibration rows)."""
    import numpy as np
    dev = W5.device
    N, K = W5.shape
    G = K // g
    Xc = X5[:calib].contiguous()
    Yref = torch.matmul(Xc, W5.t().contiguous())
    ws = torch.empty(q4.awq_workspace_bytes(calib, N, K, g, n_alpha), dtype=torch.uint8, device=dev)
    s_out = torch.empty(K, dtype=torch.float32, device=dev)
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, G), dtype=torch.float16, device=dev)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=dev)
    errors = torch.empty(n_alpha, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    run = lambda: q4.awq_search_into(Xc, Yref, W5, g, "asym", n_alpha, ws, s_out, packed, scales, zeros,
                                     errors, best)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    search_ms = e0.elapsed_time(e1) / reps
    qs = lambda: q4.quantize_rtn_scaled_into(W5, s_out, g, "asym", packed, scales, zeros)
    qs()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5 * reps):
        qs()
    e1.record()
    torch.cuda.synchronize()
    qs_ms = e0.elapsed_time(e1) / (5 * reps)
    qs_bytes = N * K * 2 + N * K // 2 + N * G * 3
    qs_gbs = qs_bytes / (qs_ms * 1e-3) / 1e9
    bi = int(best.cpu().numpy()[0])
    errs = errors.cpu().numpy()
    res = {
        "workload": f"AWQ-style scaling search, W[{N},{K}] asym g={g}, {calib} calibration rows, "
                    f"{n_alpha} alphas",
        "ms": round(search_ms, 4), "ms_per_alpha": round(search_ms / n_alpha, 4),
        "weights_alphas_per_s": round(N * K * n_alpha / (search_ms * 1e-3), 1),
        "best_alpha": round(bi / max(n_alpha - 1, 1), 3),
        "error_ratio_best_vs_rtn": round(float(errs[bi] / errs[0]), 4) if errs[0] > 0 else None,
        "quantize_scaled": {"ms": round(qs_ms, 4), "roofline": {
            "bound": "hbm", "achieved": round(qs_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(qs_gbs / HBM_PEAK_GBS, 4)}},
    }
    if with_oracle:
        from oracle import q4_oracle as orc
        from synth import f64_to_bf16_bits
        Wb = W5_bits[:oracle_rows]
        Xb = X5_bits[:oracle_calib]
        Yb = f64_to_bf16_bits(orc.bf16_bits_to_f32(Xb).astype(np.float64) @
                              orc.bf16_bits_to_f32(Wb).astype(np.float64).T)
        t = time.perf_counter()
        orc.awq_search_ref(Wb, Xb, Yb, g, "asym", n_alpha)
        spent = time.perf_counter() - t
        res["cpu_oracle"] = {"weights_alphas_per_s": round(oracle_rows * K * n_alpha / spent, 1),
                             "seconds": round(spent, 2), "kind": "oracle",
                             "sample": f"oracle awq_search_ref on the first {oracle_rows} rows of W and "
                                       f"{oracle_calib} calibration rows, {n_alpha} alphas"}
    return res


def measure_w8(torch, q4, W4, X4, W4_bits, X4_bits, X5, W5, copies=3, reps=30, with_oracle=True,
               oracle_rows=2048):
    """W8A16 (8-bit codes) on the 70B-shaped weight W[28672, 8192]: the decode GEMV at M=1,
    per-channel (g = K, the pages' W8A16) and g=128, symmetric, rotating over `copies` quantized
    copies (705 MB) so the Infinity Cache cannot serve them, and M=4; the 8-bit RTN quantizer;
    the 8-bit GEMM at the prefill shape M=2048.  HIP events on the launch stream.  Before timing,
    the GPU's codes of the first and last 64 rows are compared bit for bit with the oracle's and
    the decode outputs of those rows checked against the oracle's product (tolerance usage); these
    checks and the oracle's own timing belong to the CPU-baseline leg (skipped with
    --no-cpu-baseline)."""
    import numpy as np
    dev = W4.device
    N, K = W4.shape
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        warm_up(torch, fn)
        e0, e1 = ev(), ev()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    res = {"workload": f"W8A16 on W[{N},{K}] (70B-shaped MLP), sym; GEMM on W[{W5.shape[0]},{W5.shape[1]}] M={X5.shape[0]}"}
    usage = 0.0
    for g in (K, 128):
        G = K // g
        sets = [q4.quantize_rtn8(W4, g, "sym") for _ in range(copies)]
        torch.cuda.synchronize()
        if with_oracle:
            from oracle import q4_oracle as orc
            rows = np.r_[0:64, N - 64:N]
            ref = orc.quantize8_rtn_ref(W4_bits[rows], g, "sym")
            got = (sets[0][0].cpu().numpy()[rows], sets[0][1].cpu().view(torch.int16).numpy().view(np.uint16)[rows],
                   sets[0][2].cpu().numpy()[rows])
            for a, b in zip(got, (ref[0], ref[1].view(np.uint16), ref[2])):
                if not np.array_equal(a, b):
                    raise AssertionError(f"W8A16 quantize parity failed (g={g})")
        for M in ((1, 4) if g == 128 else (1,)):
            X = X4[:1].expand(M, K).contiguous() if M > X4.shape[0] else X4[:M].contiguous()
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fn = lambda i: q4.matmul_w8_into(X, *sets[i % copies], g, "sym", Y)
            ms = timed(fn, reps)
            by = N * K + 2 * N * G + 2 * M * K + 2 * M * N
            gbs = by / (ms * 1e-3) / 1e9
            if with_oracle:
                q4.matmul_w8_into(X, *sets[0], g, "sym", Y)
                torch.cuda.synchronize()
                Yh = Y.float().cpu().numpy().astype(np.float64)
                Xb = X.cpu().view(torch.int16).numpy().view(np.uint16)
                Yr, A = orc.matmul8_ref(Xb, ref[0], ref[1], ref[2], g, "sym")
                ok, u = orc.check_matmul(Yh[:, rows], Yr, A)
                if not ok:
                    raise AssertionError(f"W8A16 GEMV parity failed (g={g}, M={M}, usage {u})")
                usage = max(usage, u)
            key = f"gemv_g{'K' if g == K else g}_M{M}"
            res[key] = {"ms": round(ms, 5), "bytes_per_launch": by, "kernel": "gemv8_kernel",
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}
        if g == 128:
            outs = sets
            qfn = lambda i: q4.quantize_rtn8_into(W4, g, "sym", *outs[i % copies])
            qms = timed(qfn, 10)
            qby = 2 * N * K + N * K + 2 * N * G
            res["quantize_g128"] = {"ms": round(qms, 5), "bytes": qby, "roofline": {
                "bound": "hbm", "achieved": round(qby / (qms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(qby / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        del sets
    w5 = q4.quantize_rtn8(W5, 128, "sym")
    Y5 = torch.empty((X5.shape[0], W5.shape[0]), dtype=torch.bfloat16, device=dev)
    gfn = lambda i: q4.matmul_w8_into(X5, *w5, 128, "sym", Y5)
    gms = timed(gfn, 20)
    tf = 2.0 * X5.shape[0] * W5.shape[0] * W5.shape[1] / (gms * 1e-3) / 1e12
    res["gemm_g128_M2048"] = {"ms": round(gms, 4), "roofline": {
        "bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(tf / BF16_PEAK_TFLOPS, 4)}}
    if with_oracle:
        res["parity_max_tolerance_usage"] = round(usage, 4)
        from oracle import q4_oracle as orc
        Wb = W4_bits[:oracle_rows]
        t = time.perf_counter()
        c, sc, z = orc.quantize8_rtn_ref(Wb, K, "sym")
        t1 = time.perf_counter()
        orc.matmul8_ref(X4_bits[:1], c, sc, z, K, "sym")
        t2 = time.perf_counter()
        res["cpu_oracle"] = {"kind": "oracle", "sample": f"the first {oracle_rows} rows, per-channel sym",
                             "quantize_weights_per_s": round(oracle_rows * K / (t1 - t), 1),
                             "gemv_GBps_weight_bytes": round(oracle_rows * (K + 2) / (t2 - t1) / 1e9, 4)}
    return res


def measure_gemv_7b(torch, q4, reps=200, min_bytes=700e6):
    """The Llama-7B MLP up-projection decode, W[11008, 4096] asym g=128, M=1, seeded synthetic
    inputs of that workload: W4A16 GEMV over enough distinct quantized copies that the
    Infinity Cache cannot serve them, HIP events around `reps` back-to-back launches through
    the C-ABI with their arguments marshalled once (at under 10 us per launch, the Python
    binding's per-call cost would otherwise set the pace).  Beside it, the same rotation read
    by a plain streaming kernel: the practical ceiling at this size."""
    from synth import CONFIGS, make_layer
    import numpy as np
    c = CONFIGS[1]
    W_bits, X_bits = make_layer(c, M=1)
    dev = torch.device("cuda:0")
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    W, X = up(W_bits), up(X_bits)
    by = matmul_bytes(1, c.N, c.K, c.g, c.mode)
    copies = int(min_bytes // weight_bytes(c.N, c.K, c.g, c.mode)) + 1
    sets = [q4.quantize_rtn(W, c.g, c.mode) for _ in range(copies)]
    Y = torch.empty((1, c.N), dtype=torch.bfloat16, device=dev)
    lib = q4.library()
    st = torch.cuda.current_stream().cuda_stream
    args = [(X.data_ptr(), 1, c.N, c.K, c.g, q4.MODES[c.mode], p.data_ptr(), s.data_ptr(), z.data_ptr(),
             Y.data_ptr(), st) for (p, s, z) in sets]
    for a in args:
        assert lib.q4_matmul(*a) == 0
    warm_up(torch, lambda r: lib.q4_matmul(*args[r % copies]))   # untimed: the same launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        lib.q4_matmul(*args[r % copies])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = by / (ms * 1e-3) / 1e9
    out = {"workload": f"{c.name}, {copies} weight copies", "kernel": q4.select_kernel(1, c.N, c.K, c.g),
           "ms": round(ms, 5), "bytes_per_launch": by,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    # the practical ceiling at this size: a plain streaming read of each copy's packed codes,
    # back to back over the same rotation (best of a few grid sizes)
    import ctypes
    from weight_only_int4_group_amd.build import BENCH_LIB
    if os.path.exists(BENCH_LIB):
        blib = ctypes.CDLL(BENCH_LIB)
        blib.q4b_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p]
        blib.q4b_stream_read.restype = ctypes.c_int
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        sink = torch.empty(cus * 64 * 4, dtype=torch.int32, device=dev)
        nb = sets[0][0].numel()
        best = None
        for per_cu in (2, 4, 8, 16, 32):
            run = [(p.data_ptr(), nb, sink.data_ptr(), cus * per_cu, st) for (p, _, _) in sets]
            warm_up(torch, lambda r: blib.q4b_stream_read(*run[r % copies]))
            e0.record()
            for r in range(reps):
                blib.q4b_stream_read(*run[r % copies])
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps
            if best is None or t < best[0]:
                best = (t, per_cu)
        rgbs = nb / (best[0] * 1e-3) / 1e9
        out["stream_read_same_size"] = {"GB/s": round(rgbs, 1), "frac": round(rgbs / HBM_PEAK_GBS, 4),
                                        "us": round(best[0] * 1e3, 2), "bytes": nb, "blocks_per_cu": best[1],
                                        "how": "libq4_bench stream_read over each copy's packed codes, "
                                               "rotating as the GEMV does; best of 2-32 blocks per CU"}
    return out


def measure_decode_range(torch, q4, reps=300, min_bytes=700e6):
    """The M <= 16 decode workloads, each on its seeded synthetic inputs (synth recipe): config 1
    (tiny 128 x 256, M=1, a launch-latency case: time reported), config 3 (batched decode
    4096 x 4096, M=16, sym), config 4 at M = 4 and 8 (70B-shaped MLP) and the 70B shape at M=16;
    beside them the 70B shape at M = 32 (the decode kernel in two 16-row launches) and 64 (the
    GEMM), the batch sizes between decode and prefill.
    Each rotates over enough distinct quantized weight copies that the Infinity Cache cannot
    serve them; the kernel q4_matmul picks (Q4_KERNEL_AUTO) is launched `reps` times back to back
    through the C-ABI with its arguments marshalled once, between HIP events on the launch
    stream.  Algorithmic bytes per launch = packed codes + fp16 scales + uint8 zeros (asym) + X
    + Y; the roofline is HBM."""
    from synth import CONFIGS, make_layer
    import numpy as np
    dev = torch.device("cuda:0")
    lib = q4.library()
    st = torch.cuda.current_stream().cuda_stream
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    import dataclasses
    c4 = CONFIGS[3]
    c4_16 = dataclasses.replace(c4, M_max=16)     # the config-4 recipe drawn with 16 rows of X
    c4_64 = dataclasses.replace(c4, M_max=64)     # ... and with 64 (mid-range batches)
    cases = [("config1", CONFIGS[0], 1), ("config3", CONFIGS[2], 16), ("config4_m4", c4, 4),
             ("config4_m8", c4, 8), ("70b_m16", c4_16, 16), ("70b_m32", c4_64, 32), ("70b_m64", c4_64, 64)]
    out = {}
    drawn = {}
    for key, c, M in cases:
        if c not in drawn:                          # one draw per recipe; M = 4 nests in M = 8
            drawn[c] = make_layer(c)
        W_bits, X_bits = drawn[c]
        W, X = up(W_bits), up(X_bits[:M])
        by = matmul_bytes(M, c.N, c.K, c.g, c.mode)
        copies = max(1, int(min_bytes // weight_bytes(c.N, c.K, c.g, c.mode)) + 1)
        copies = min(copies, 400)
        sets = [q4.quantize_rtn(W, c.g, c.mode) for _ in range(copies)]
        del W
        Y = torch.empty((M, c.N), dtype=torch.bfloat16, device=dev)
        args = [(X.data_ptr(), M, c.N, c.K, c.g, q4.MODES[c.mode], p.data_ptr(), s.data_ptr(), z.data_ptr(),
                 Y.data_ptr(), st) for (p, s, z) in sets]
        for a in args:
            assert lib.q4_matmul(*a) == 0
        warm_up(torch, lambda r: lib.q4_matmul(*args[r % copies]))   # untimed: the same launches
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            lib.q4_matmul(*args[r % copies])
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = by / (ms * 1e-3) / 1e9
        out[key] = {"workload": f"{c.name}" + (f" at M={M}" if M != c.M_max else "") + f", {copies} weight copies",
                    "M": M, "N": c.N, "K": c.K, "g": c.g, "mode": c.mode,
                    "kernel": q4.select_kernel(M, c.N, c.K, c.g), "ms": round(ms, 5), "bytes_per_launch": by,
                    "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}
        del sets, args
        torch.cuda.empty_cache()
    return out


def measure_gptq(torch, q4, W5, X5, W5_bits, X5_bits, calib=512, g=128, reps=3, with_oracle=True,
                 oracle_rows=32):
    """GPTQ of the prefill layer W[8192, 8192] (asym, g=128) on `calib` calibration rows of its
    activations: q4_gptq timed with HIP events on the launch stream.  Algorithmic flops:
    M K^2 for H = X^T X (its lower half), K^3 / 3 for the Cholesky factorisation and N K^2 for
    the error-feedback sweep (sum over columns of 2 N i).  The oracle's gptq_ref is timed beside
    it on a bounded sample (`oracle_rows` rows of W; its Hessian factorisation is full size)."""
    import numpy as np
    dev = W5.device
    N, K = W5.shape
    G = K // g
    Xc = X5[:calib].contiguous()
    ws = torch.empty(q4.gptq_workspace_bytes(calib, N, K, g), dtype=torch.uint8, device=dev)
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, G), dtype=torch.float16, device=dev)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    run = lambda: q4.gptq_into(Xc, W5, g, "asym", 0.01, ws, packed, scales, zeros, info)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = calib * K * K + K ** 3 / 3 + N * K * K
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": f"GPTQ of W[{N},{K}] asym g={g} on {calib} calibration rows (damp 0.01)",
           "ms": round(ms, 3), "info": int(info.cpu().numpy()[0]), "flops": flops,
           "roofline": {"bound": "alu", "achieved": round(tf, 2), "peak": FP32_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / FP32_PEAK_TFLOPS, 4)}}
    if with_oracle:
        from oracle import q4_oracle as orc
        t = time.perf_counter()
        orc.gptq_ref(W5_bits[:oracle_rows], X5_bits[:calib], g, "asym")
        spent = time.perf_counter() - t
        res["cpu_oracle"] = {"kind": "oracle", "seconds": round(spent, 2),
                             "sample": f"oracle gptq_ref on the first {oracle_rows} rows of W with the full "
                                       f"{K} x {K} Hessian ({calib} calibration rows)",
                             "rows_per_s": round(oracle_rows / spent, 2),
                             "gpu_rows_per_s": round(N / (ms * 1e-3), 1)}
    return res


def measure_dequant(torch, q4, sets, W4_bits, g=128, reps=30, with_oracle=True, oracle_rows=1024):
    """q4_dequantize of the 70B-shaped weight W[28672, 8192] (asym, g=128) to bf16, rotating over
    the benchmark's per-layer quantized copies; algorithmic bytes = codes + scales + zeros read + the
    bf16 output written.  In the CPU-baseline leg the oracle quantizes the first `oracle_rows`
    rows, the library dequantizes those codes and must match the oracle's dequantization bit
    for bit, and the oracle's dequantization is timed."""
    import numpy as np
    p0 = sets[0][0]
    N, K = p0.shape[0], p0.shape[1] * 2
    G = K // g
    out = torch.empty((N, K), dtype=torch.bfloat16, device=p0.device)
    L = len(sets)
    run = lambda i: q4.dequantize_into(*sets[i % L], g, "asym", out)
    run(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    by = N * K // 2 + 3 * N * G + 2 * N * K
    gbs = by / (ms * 1e-3) / 1e9
    res = {"workload": f"q4_dequantize of W[{N},{K}] asym g={g} to bf16, {L} weight copies",
           "ms": round(ms, 5), "bytes_per_launch": by, "kernel": "dequant_kernel",
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    if with_oracle:
        from oracle import q4_oracle as orc
        rp, rs, rz = orc.quantize_rtn_ref(W4_bits[:oracle_rows], g, "asym")
        dev = p0.device
        pd = torch.from_numpy(rp).to(dev)
        sd = torch.from_numpy(rs.view(np.int16)).view(torch.float16).to(dev)
        zd = torch.from_numpy(rz).to(dev)
        got = q4.dequantize(pd, sd, zd, g, "asym")
        torch.cuda.synchronize()
        t = time.perf_counter()
        want = orc.dequantize_rounded_ref(rp, rs, rz, g, "asym", "bf16")
        spent = time.perf_counter() - t
        if not np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), want):
            raise AssertionError("dequantize parity failed")
        res["cpu_oracle"] = {"kind": "oracle", "sample": f"oracle dequantize_rounded_ref of the first "
                                                          f"{oracle_rows} rows (bf16 out)",
                             "seconds": round(spent, 3),
                             "GB/s": round(oracle_rows * (K // 2 + 3 * G + 2 * K) / spent / 1e9, 4)}
    return res


# --------------------------------------------------------------------------- counters
def _counter_rows(d):
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def measured_clocks(d):
    """Shader clock during the prefill GEMM: GRBM_GUI_ACTIVE (GPU-busy cycles, summed over the
    XCDs) / number of XCDs / dispatch duration, from a counter run that collected
    GRBM_GUI_ACTIVE.  (For a kernel of a few tens of microseconds the counter window's own
    busy time dominates, so the decode kernels get no such figure.)"""
    xcc = 1
    for path in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Name", "").startswith("gfx") and int(r.get("Num_Xcc") or 0) > 0:
                    xcc = int(r["Num_Xcc"])
    out = {}
    for label, key in (("prefill", "prefill_kernel<256"),):
        cyc, ns = [], []
        for r in _counter_rows(d):
            if r.get("Counter_Name") == "GRBM_GUI_ACTIVE" and key in r.get("Kernel_Name", ""):
                cyc.append(float(r["Counter_Value"]))
                ns.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        if cyc:
            ghz = sum(c / xcc / t for c, t in zip(cyc, ns)) / len(cyc)
            out[f"{label}_clock_GHz"] = round(ghz, 3)
            out[f"{label}_clock_dispatches"] = len(cyc)
    return out


def summarize_counters(fetch_dir, write_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the GEMV, scaled by a plain copy's.

    The calibration copy is the one device-to-device copy of 512 MiB that
    ``--copy-calibration`` launches: the copy dispatch whose WRITE_SIZE is closest to 512 MiB
    (its FETCH_SIZE is taken from the same dispatch index of the other run).
    """
    def per_kernel(d, counter):
        out = {}
        for r in _counter_rows(d):
            if r.get("Counter_Name") != counter:
                continue
            out.setdefault(r.get("Kernel_Name", ""), []).append(float(r["Counter_Value"]))
        return out

    def mean_of(d, key):
        vals = [x for k, v in d.items() if key(k) for x in v]
        return (sum(vals) / len(vals), len(vals)) if vals else None

    copy_bytes = 512 * 2 ** 20
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    is_gemv = lambda k: "gemv_kernel<1, 4," in k          # the 70B-shaped M = 1 instance
    is_copy = lambda k: "copyBuffer" in k
    gf, gw = mean_of(fetch, is_gemv), mean_of(write, is_gemv)
    cw_all = [x for k, v in write.items() if is_copy(k) for x in v]
    cf_all = [x for k, v in fetch.items() if is_copy(k) for x in v]
    cw = cf = None
    if cw_all and cf_all and len(cw_all) == len(cf_all):
        i = min(range(len(cw_all)), key=lambda j: abs(cw_all[j] * 1024 - copy_bytes))
        cw, cf = cw_all[i], cf_all[i]
    res = {
        "gemv_src_sha": src_sha(GEMV_SRC),
        "gemv_fetch_kib_per_dispatch": gf[0] if gf else None,
        "gemv_write_kib_per_dispatch": gw[0] if gw else None,
        "gemv_dispatches": gf[1] if gf else 0,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": cf,
        "copy_write_kib": cw,
    }
    res.update(measured_clocks(fetch_dir))
    if gf and gw and cf and cw:
        ff = copy_bytes / (cf * 1024)
        fw = copy_bytes / (cw * 1024)
        res["copy_factor_fetch"] = ff
        res["copy_factor_write"] = fw
        res["traffic_bytes_per_launch"] = gf[0] * 1024 * ff + gw[0] * 1024 * fw
        # every kernel of the run, scaled the same way (MB per dispatch)
        res["per_kernel_MB"] = {
            k: {"fetch": round(sum(v) / len(v) * 1024 * ff / 1e6, 3),
                "write": round(sum(write.get(k, [0.0])) / max(1, len(write.get(k, []))) * 1024 * fw / 1e6, 3),
                "dispatches": len(v)}
            for k, v in sorted(fetch.items())}
    else:
        res["traffic_bytes_per_launch"] = None
    return res


def summarize_trace(trace_dir):
    """Per-kernel dispatch count and duration statistics (us) from rocprofv3 kernel-trace
    csv files: mean, median, p10, p90, min, max, sorted by total time."""
    import statistics
    durs = {}
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                durs.setdefault(r["Kernel_Name"], []).append(d)

    def pct(v, q):
        v = sorted(v)
        i = q * (len(v) - 1)
        lo = int(i)
        hi = min(lo + 1, len(v) - 1)
        return v[lo] + (v[hi] - v[lo]) * (i - lo)

    rows = []
    for name, v in durs.items():
        rows.append({"kernel": name, "calls": len(v), "total_us": round(sum(v), 1),
                     "mean_us": round(sum(v) / len(v), 2), "median_us": round(statistics.median(v), 2),
                     "p10_us": round(pct(v, 0.1), 2), "p90_us": round(pct(v, 0.9), 2),
                     "min_us": round(min(v), 2), "max_us": round(max(v), 2)})
    rows.sort(key=lambda r: -r["total_us"])
    return rows


# --------------------------------------------------------------------------- workload
def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W_bits, X_bits, g, mode, budget_s=10.0, q_budget_s=6.0, block=4096, W5_bits=None,
                 X5_bits=None, prefill_rows=256):
    """The CPU oracle, timed on this host over bounded samples of the 70B-shaped layer.

    matmul_ref (M=1, fp64 dequantisation + BLAS, all BLAS threads): the oracle quantizes each
    row block first (not timed), then matmul_ref is timed over the blocks, cycling through the
    layer until about budget_s seconds are spent.  quantize_ref (elementwise numpy, one
    thread) is timed on consecutive row blocks until about q_budget_s seconds are spent.  The
    prefill product (M = 2048) is timed on `prefill_rows` rows of the prefill layer's W.
    """
    import numpy as np
    from oracle import q4_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    N, K = W_bits.shape
    blocks = [orc.quantize_rtn_ref(W_bits[r:r + block], g, mode) for r in range(0, N, block)]
    done_rows, spent, passes = 0, 0.0, 0
    while spent < budget_s:
        for p, s, z in blocks:
            t = time.perf_counter()
            orc.matmul_ref(X_bits, p, s, z, g, mode)
            spent += time.perf_counter() - t
            done_rows += p.shape[0]
        passes += 1
    nbytes = matmul_bytes(X_bits.shape[0], done_rows, K, g, mode)
    q_rows, q_spent, qb = 0, 0.0, 512
    while q_spent < q_budget_s and q_rows < N:
        t = time.perf_counter()
        orc.quantize_rtn_ref(W_bits[q_rows:q_rows + qb], g, mode)
        q_spent += time.perf_counter() - t
        q_rows += min(qb, N - q_rows)
    G = K // g
    q_bytes = q_rows * (2 * K + K // 2 + G * (3 if mode == "asym" else 2))
    prefill = None
    if W5_bits is not None:
        p5, s5, z5 = orc.quantize_rtn_ref(W5_bits[:prefill_rows], 128, "asym")
        t = time.perf_counter()
        orc.matmul_ref(X5_bits, p5, s5, z5, 128, "asym")
        ps = time.perf_counter() - t
        prefill = {"TFLOP/s": round(2.0 * X5_bits.shape[0] * prefill_rows * W5_bits.shape[1] / ps / 1e12, 5),
                   "seconds": round(ps, 3),
                   "sample": f"oracle matmul_ref, M={X5_bits.shape[0]}, the first {prefill_rows} rows of the "
                             f"prefill layer's W (g=128 asym)"}
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "prefill_matmul_ref": prefill,
            "kind": "oracle",
            "sample": f"oracle matmul_ref (fp64 dequantisation + BLAS), M=1, the whole {N}x{K} "
                      f"layer in row blocks of {block}, {passes} passes, {spent:.1f} s",
            "cpu_model": cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
            "gflops": round(2.0 * done_rows * K / spent / 1e9, 3),
            "quantize_ref": {"GB/s": round(q_bytes / q_spent / 1e9, 4), "cores": 1,
                             "sample": f"oracle quantize_rtn_ref (elementwise numpy fp32), first {q_rows} rows "
                                       f"of the {N}x{K} weight in blocks of {qb}, {q_spent:.1f} s; bytes = "
                                       f"bf16 W read + codes, scales, zeros written"}}


def check_parity(q4, torch, W4_bits, X4_bits, sets, Y4, W5_bits, X5_host, X5_dev, w5, Y5):
    """Sampled parity of every timed kernel against the oracle (asserts)."""
    import numpy as np
    from oracle import q4_oracle as orc
    rng = np.random.default_rng(7)
    # quantize: sampled rows bit-exact
    rows = np.sort(rng.choice(W4_bits.shape[0], 256, replace=False))
    rp, rs, rz = orc.quantize_rtn_ref(W4_bits[rows], 128, "asym")
    p, s, z = sets[0]
    assert np.array_equal(p[rows].cpu().numpy(), rp), "quantize: packed differs"
    assert np.array_equal(s[rows].cpu().view(torch.int16).numpy().view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(z[rows].cpu().numpy(), rz), "quantize: zeros differ"
    # decode GEMV on copy 0 (bit-identical to the oracle's weights on the sampled rows)
    q4.matmul_into(torch.from_numpy(X4_bits.view(np.int16)).view(torch.bfloat16).cuda(), p, s, z,
                   128, "asym", Y4)
    torch.cuda.synchronize()
    Y = Y4.float().cpu().numpy().astype(np.float64)
    Yr, A = orc.matmul_ref(X4_bits, rp, rs, rz, 128, "asym")
    ok, u1 = orc.check_matmul(Y[:, rows], Yr, A)
    assert ok, f"GEMV outside tolerance (usage {u1})"
    # GEMM: sampled entries, weights re-quantized by the oracle on the sampled rows
    usages = [u1]
    for g, (p5, s5, z5) in w5.items():
        q4.matmul_into(X5_dev, p5, s5, z5, g, "asym", Y5)
        torch.cuda.synchronize()
        n_idx = np.sort(rng.choice(W5_bits.shape[0], 64, replace=False))
        m_idx = rng.choice(X5_host.shape[0], 64, replace=False)
        rp5, rs5, rz5 = orc.quantize_rtn_ref(W5_bits[n_idx], g, "asym")
        assert np.array_equal(p5[n_idx].cpu().numpy(), rp5)
        Yr5, A5 = orc.matmul_ref(X5_host[m_idx], rp5, rs5, rz5, g, "asym")
        Yg = Y5[m_idx][:, n_idx].float().cpu().numpy().astype(np.float64)
        ok, u = orc.check_matmul(Yg, Yr5, A5)
        assert ok, f"GEMM g={g} outside tolerance (usage {u})"
        usages.append(u)
    return max(usages)


def main(argv=None):
    args = parse_args(argv)
    if args.summarize_counters:
        res = summarize_counters(*args.summarize_counters)
        print(json.dumps(res, indent=1))
        return 0
    if args.summarize_trace:
        for r in summarize_trace(args.summarize_trace):
            print(json.dumps(r))
        return 0
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the path is single-GPU; sharding is "
              "described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import weight_only_int4_group_amd as q4
    from synth import CONFIGS, make_layer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    c4, c5 = CONFIGS[3], CONFIGS[4]
    N4, K4, g4 = c4.N, c4.K, c4.g
    W4_bits, X4_bits = make_layer(c4, M=1)
    W5_bits, X5_bits = make_layer(c5)
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    W4, X4 = up(W4_bits), up(X4_bits)
    W5, X5 = up(W5_bits), up(X5_bits)
    G4 = K4 // g4
    L = args.layers
    sets = [(torch.empty((N4, K4 // 2), dtype=torch.uint8, device=dev),
             torch.empty((N4, G4), dtype=torch.float16, device=dev),
             torch.empty((N4, G4), dtype=torch.uint8, device=dev)) for _ in range(L)]
    for s in sets:
        q4.quantize_rtn_into(W4, g4, "asym", *s)
    w5L = {g: [q4.quantize_rtn(W5, g, "asym") for _ in range(L)] for g in (128, 32)}
    w5 = {g: w5L[g][0] for g in w5L}
    Y4 = torch.empty((1, N4), dtype=torch.bfloat16, device=dev)
    Y5 = torch.empty((X5.shape[0], c5.N), dtype=torch.bfloat16, device=dev)
    copy_src = copy_dst = None
    if args.copy_calibration:
        copy_src = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev).fill_(1)
        copy_dst = torch.empty_like(copy_src)
    torch.cuda.synchronize()

    # The parity assertion is part of the CPU-baseline leg: the oracle runs only there.
    note("inputs ready")
    max_usage = None
    if not args.no_check and not args.no_cpu_baseline:
        max_usage = check_parity(q4, torch, W4_bits, X4_bits, sets, Y4, W5_bits, X5_bits, X5, w5, Y5)
        note("parity checked against the oracle")

    n_ev = 5
    def step(t, ev):
        ev[0].record()
        q4.quantize_rtn_into(W4, g4, "asym", *sets[t % L])
        ev[1].record()
        for i in range(L):
            p, s, z = sets[(t + 1 + i) % L]
            q4.matmul_into(X4, p, s, z, g4, "asym", Y4)
        ev[2].record()
        for i in range(L):
            q4.matmul_into(X5, *w5L[128][(t + i) % L], 128, "asym", Y5)
        ev[3].record()
        for i in range(L):
            q4.matmul_into(X5, *w5L[32][(t + i) % L], 32, "asym", Y5)
        ev[4].record()

    warm = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(max(args.warmup, 0))]
    for t in range(args.warmup):
        step(t, warm[t])
    if copy_dst is not None:
        copy_dst.copy_(copy_src)
    torch.cuda.synchronize()

    # The timed region runs the same K passes of the path phase-major: every phase's launches go
    # back to back between one pair of events, as a decode loop runs its layers.  (An event pair
    # between individual launches costs a few microseconds of its own on this stack, which would
    # be charged to the 22-us GEMV.)
    K_ = args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for t in range(K_):
        q4.quantize_rtn_into(W4, g4, "asym", *sets[(args.warmup + t) % L])
    evs[1].record()
    for t in range(K_):
        for i in range(L):
            p, s, z = sets[(args.warmup + t + 1 + i) % L]
            q4.matmul_into(X4, p, s, z, g4, "asym", Y4)
    evs[2].record()
    for t in range(K_):
        for i in range(L):
            q4.matmul_into(X5, *w5L[128][(args.warmup + t + i) % L], 128, "asym", Y5)
    evs[3].record()
    for t in range(K_):
        for i in range(L):
            q4.matmul_into(X5, *w5L[32][(args.warmup + t + i) % L], 32, "asym", Y5)
    evs[4].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    note(f"{args.steps} timed steps done")

    def mean_ms(i, j):
        return evs[i].elapsed_time(evs[j]) / K_

    q_ms = mean_ms(0, 1)
    gemv_ms = mean_ms(1, 2) / L
    g128_ms = mean_ms(2, 3) / L
    g32_ms = mean_ms(3, 4) / L

    gemv_bytes = matmul_bytes(1, N4, K4, g4, "asym")
    gemv_gbs = gemv_bytes / (gemv_ms * 1e-3) / 1e9
    flops = 2.0 * X5.shape[0] * c5.N * c5.K
    g128_tf = flops / (g128_ms * 1e-3) / 1e12
    g32_tf = flops / (g32_ms * 1e-3) / 1e12
    q_bytes = quantize_bytes(N4, K4, g4)
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    traffic = read_traffic()

    out = {
        "metric": METRIC,
        "value": round(gemv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"70B-shaped MLP decode: W4A16 GEMV M=1, W[{N4},{K4}] asym g={g4}, "
                         f"{L} layers per step, each with its own weight copy; plus RTN quantize "
                         f"of that W and prefill GEMM M={X5.shape[0]} W[{c5.N},{c5.K}] g=128 and "
                         f"g=32 through the same {L} layers"),
            "M": 1, "N": N4, "K": K4, "g": g4, "mode": "asym", "layers_per_step": L,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(gemv_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else int(traffic),
            "kernel": "gemv_kernel", "bytes_per_launch": gemv_bytes,
            "ms_per_launch": round(gemv_ms, 5),
        },
        "gemm": {
            "M": int(X5.shape[0]), "N": c5.N, "K": c5.K,
            "g128": {"tflops": round(g128_tf, 2), "ms": round(g128_ms, 4),
                     "roofline": {"bound": "mfma", "achieved": round(g128_tf, 2),
                                  "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(g128_tf / BF16_PEAK_TFLOPS, 4)}},
            "g32": {"tflops": round(g32_tf, 2), "ms": round(g32_ms, 4),
                    "roofline": {"bound": "mfma", "achieved": round(g32_tf, 2),
                                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(g32_tf / BF16_PEAK_TFLOPS, 4)}},
        },
        "quantize": {"GB/s": round(q_gbs, 2), "ms": round(q_ms, 4), "bytes": q_bytes,
                     "roofline": {"bound": "hbm", "achieved": round(q_gbs, 2), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(q_gbs / HBM_PEAK_GBS, 4)}},
        "parity_max_tolerance_usage": max_usage,
    }
    if not args.no_context:
        out["context"] = measure_context(torch, q4, sets, X5, W5, w5)
        note("context measured")
    out["dequantize"] = measure_dequant(torch, q4, sets, W4_bits, with_oracle=not args.no_cpu_baseline)
    note("standalone dequantize measured")
    out["gemv_llama7b_up"] = measure_gemv_7b(torch, q4)
    note("Llama-7B-shaped decode measured")
    out["decode_m_le_16"] = measure_decode_range(torch, q4)
    note("M <= 16 decode workloads measured")
    if not args.no_w8:
        out["w8a16"] = measure_w8(torch, q4, W4, X4, W4_bits, X4_bits, X5, W5,
                                  with_oracle=not args.no_cpu_baseline)
        note("W8A16 measured")
    if not args.no_gptq:
        out["gptq"] = measure_gptq(torch, q4, W5, X5, W5_bits, X5_bits, with_oracle=not args.no_cpu_baseline)
        note("GPTQ measured")
    if not args.no_awq:
        out["awq"] = measure_awq(torch, q4, W5, X5, W5_bits, X5_bits, with_oracle=not args.no_cpu_baseline)
        note("AWQ search measured")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W4_bits, X4_bits, g4, "asym", W5_bits=W5_bits, X5_bits=X5_bits)
        note("CPU baseline timed")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
