"""Host-side checks of the benchmark contract: one GPU only, algorithmic
bytes counted at the codes' bit width, and the committed HBM-traffic
summaries that bench.py reads for roofline.traffic self-consistent (no GPU
needed)."""
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bench_workloads as bw  # noqa: E402
import workloads as wl  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_at_code_width():
    M, K, N = 4096, 3072, 3072
    # rotate+quantize: bf16 in, 4 or 8 bits per code out, plus the scales
    assert bw.rq_bytes(M, K, "int4_tensor") == 2 * M * K + M * K // 2 + 4
    assert bw.rq_bytes(M, K, "int8_tensor") == 2 * M * K + M * K + 4
    assert bw.rq_bytes(M, K, "dual_tensor") == 2 * M * K + M * K // 2 + M * K + 8
    assert bw.rq_bytes(M, K, "int8_row_f16") == 2 * M * K + M * K + 4 * M
    # GEMM: codes and weights at 4 bits (INT4) or 8 bits (INT8), bf16 output
    lin = wl.LinearSpec("p", "w4a4", M, N, K, "x")
    assert bw.gemm_bytes(lin) == M * K // 2 + N * K // 2 + 2 * M * N
    lin8 = wl.LinearSpec("p", "int8", M, N, K, "x")
    assert bw.gemm_bytes(lin8) == M * K + N * K + 2 * M * N


def test_side_line_roofline_bounds():
    """Each format is priced against what bounds it: weight bytes at small M,
    one float32 FMA per output and group on the vector ALUs (78.6 TFLOP/s
    without packed math) for W4A8 and the 64-group format, else the matrix
    cores of its operand type."""
    assert abs(bw.VALU_FP32_TFLOPS - 256 * 4 * 16 * 2 * 2.4e9 / 1e12) < 0.05
    w4a8 = wl.LinearSpec("p", "w4a8", 8192, 12288, 3072, "x")
    r = bw.gemm_roofline(w4a8, 600.0)
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - 2 * 8192 * 12288 * 192 / 600e-6 / 1e12) < 0.1
    g64 = wl.LinearSpec("p", "w4a4_g64", 8192, 3072, 12288, "x")
    assert bw.gemm_roofline(g64, 300.0)["achieved"] == round(2 * 8192 * 3072 * 192 / 300e-6 / 1e12, 1)
    f6 = wl.LinearSpec("p", "w4a4", 4096, 3072, 3072, "x")
    r = bw.gemm_roofline(f6, 30.0)
    assert r["bound"] == "mfma" and r["peak"] == bw.FP6_PEAK_TOPS
    assert bw.gemm_roofline(f6, 30.0, cores="int8")["peak"] == bw.INT8_PEAK_TOPS
    a8 = wl.LinearSpec("p", "a8w4", 4096, 3072, 3072, "x")
    assert bw.gemm_roofline(a8, 70.0)["peak"] == bw.INT8_PEAK_TOPS
    small = wl.LinearSpec("p", "w4a4", 32, 3072, 3072, "x")
    r = bw.gemm_roofline(small, 4.0)
    assert r["bound"] == "hbm" and r["achieved"] == round(bw.gemm_bytes(small) / 4.0 / 1e3, 1)


def test_c4_plan_matches_the_recipe():
    # 14 linears; W4A4: q, k, mlp_up, mlp_down; INT8: v, out, mod (both streams);
    # the attention input is quantized once for the INT4 and INT8 layers
    w = wl.CONFIGS["c4"]()
    rq, gemms = bw.plan(w)
    assert len(gemms) == 14
    fmts = {l.name: l.fmt for l in w.linears}
    for s in ("img", "txt"):
        assert [fmts[f"{s}_{n}"] for n in ("q", "k", "mlp_up", "mlp_down")] == ["w4a4"] * 4
        assert [fmts[f"{s}_{n}"] for n in ("v", "out", "mod")] == ["int8"] * 3
        assert (f"{s}_attn", "dual_tensor", "") in rq
    assert abs(sum(2.0 * l.M * l.N * l.K for l in w.linears) / 1e9 - 1971.8) < 0.1


def test_traffic_profiles_consistent():
    for p in glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")):
        with open(p) as f:
            d = json.load(f)
        assert d["hbm_bytes_per_launch"] == d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]
        M, N, K = d["M"], d["N"], d["K"]
        lin = wl.LinearSpec(d["layer"], d["fmt"], M, N, K, "x")
        assert d["algorithmic_bytes_per_launch"] == int(bw.gemm_bytes(lin))
        # every launch writes at least its bf16 output and reads at least its operands once
        assert d["write_bytes_per_launch"] >= 0.99 * 2 * M * N
        assert len(d["source_sha"]) == 16
        cores = d["cores"]
        if d["source_sha"] == bench.source_sha(bench.GEMM_SOURCES[cores]):
            assert bench.traffic_from_profile(cores, d["layer"]) == d["hbm_bytes_per_launch"]
        else:
            assert bench.traffic_from_profile(cores, d["layer"]) is None


def test_shader_clock_without_a_gpu():
    """With no GPU the management library finds no device: the clock reading
    is None and nothing is launched."""
    calls = []

    class NoGpu:
        torch = None
        stream = None

    assert bw.Runner.shader_clock(NoGpu(), calls.append, 50) is None
    assert calls == []


def test_fuse_shared_inputs_merges_only_same_input_w4a4_runs():
    """The block's Q and K projections (same input, shape, chain and phase,
    W4A4) become one layer with both weights side by side; every other layer
    stays as defined; the work, the inputs and the defined parts are kept."""
    w = wl.CONFIGS["c4"]()
    f = bw.fuse_shared_inputs(w)
    names = [l.name for l in f.linears]
    assert names == ["img_q+img_k", "img_v", "img_out", "img_mlp_up", "img_mlp_down", "img_mod",
                     "txt_q+txt_k", "txt_v", "txt_out", "txt_mlp_up", "txt_mlp_down", "txt_mod"]
    qk = f.linears[0]
    assert (qk.M, qk.N, qk.K, qk.x_id, qk.chain, qk.phase) == (8192, 6144, 3072, "img_attn", "img", 0)
    assert [p.name for p in qk.parts] == ["img_q", "img_k"] and all(p in w.linears for p in qk.parts)
    assert sum(2 * l.M * l.N * l.K for l in f.linears) == sum(2 * l.M * l.N * l.K for l in w.linears)
    assert f.acts == w.acts and f.config_id == w.config_id
    # the weights of every defined linear are drawn as in the defined workload
    assert all(not l.parts for l in w.linears)
    # nothing to merge elsewhere: a single W4A4 layer, the low-rank format, INT8 layers
    for name in ("c2", "c3", "c5"):
        d = wl.CONFIGS[name]()
        assert [l.name for l in bw.fuse_shared_inputs(d).linears] == [l.name for l in d.linears]
    # the RQ plan is unchanged: one dual pass per stream's attention input
    assert bw.plan(f)[0] == bw.plan(w)[0]
