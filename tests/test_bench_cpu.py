"""Host-side checks of the benchmark contract: one GPU only, and the
committed HBM-traffic summaries that bench.py reads for roofline.traffic
are self-consistent (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("cores", ["fp6", "int8"])
def test_traffic_profiles_consistent(cores):
    with open(os.path.join(ROOT, "profiles", bench.TRAFFIC_PROFILE[cores])) as f:
        d = json.load(f)
    M, N, K = 4096, 3072, 3072
    code_bytes = 0.75 if cores == "fp6" else 0.5
    # algorithmic bytes: activation codes + packed weights + bf16 output
    assert d["algorithmic_bytes_per_launch"] == int(M * K * code_bytes + N * K * code_bytes + 2 * M * N)
    assert d["hbm_bytes_per_launch"] == d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]
    # every launch writes at least its bf16 output and reads at least its operands once
    assert d["write_bytes_per_launch"] >= 0.99 * 2 * M * N
    assert d["fetch_bytes_per_launch"] >= 0.99 * (M * K + N * K) * code_bytes
    assert len(d["source_sha"]) == 16
    # bench.py uses the summary only while the kernel sources hash the same
    bench.CORES = cores
    t = bench.traffic_from_profile()
    if d["source_sha"] == bench.source_sha(bench.GEMM_SOURCES[cores]):
        assert t == d["hbm_bytes_per_launch"]
    else:
        assert t is None
