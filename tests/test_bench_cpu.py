"""Host logic of bench.py, without a GPU: the one-GPU contract, the algorithmic byte counts that
the rooflines divide by, and the rocprofv3 trace summary."""
import csv
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line for a configuration that is not measured


def _storage(N, K, g, mode):
    """The arrays of the storage format, as the library's outputs hold them."""
    G = K // g
    arrs = [np.zeros((N, K // 2), np.uint8), np.zeros((N, G), np.float16)]
    if mode == "asym":
        arrs.append(np.zeros((N, G), np.uint8))
    return arrs


def test_weight_and_matmul_bytes_count_every_array_once():
    for (M, N, K, g, mode) in [(1, 28672, 8192, 128, "asym"), (2048, 8192, 8192, 32, "asym"),
                               (4, 11008, 4096, 128, "sym"), (1, 96, 384, 96, "asym")]:
        w = sum(a.nbytes for a in _storage(N, K, g, mode))
        assert bench.weight_bytes(N, K, g, mode) == w
        x = np.zeros((M, K), np.uint16).nbytes
        y = np.zeros((M, N), np.uint16).nbytes
        assert bench.matmul_bytes(M, N, K, g, mode) == w + x + y
    # the headline layer: 123.02 MB per decode launch
    assert bench.matmul_bytes(1, 28672, 8192, 128, "asym") == 123_019_264


def test_quantize_bytes_read_bf16_write_the_format():
    N, K, g = 28672, 8192, 128
    w_in = np.zeros((N, K), np.uint16).nbytes
    out = sum(a.nbytes for a in _storage(N, K, g, "asym"))
    assert bench.quantize_bytes(N, K, g) == w_in + out


def test_summarize_trace_statistics(tmp_path):
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    rows = []
    t = 1_000_000
    durs_a = [10.0, 20.0, 30.0, 40.0, 50.0]          # us
    durs_b = [100.0, 300.0]
    for name, durs in (("kernel_a", durs_a), ("kernel_b", durs_b)):
        for us in durs:
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + int(us * 1000)})
            t += 10_000_000
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    out = bench.summarize_trace(str(tmp_path / "trace"))
    assert [r["kernel"] for r in out] == ["kernel_b", "kernel_a"]          # by total time
    b, a = out
    assert (a["calls"], a["total_us"], a["mean_us"], a["median_us"]) == (5, 150.0, 30.0, 30.0)
    assert (a["p10_us"], a["p90_us"], a["min_us"], a["max_us"]) == (14.0, 46.0, 10.0, 50.0)
    assert (b["calls"], b["mean_us"], b["median_us"], b["p10_us"], b["p90_us"]) == (2, 200.0, 200.0, 120.0, 280.0)
