"""Benchmark of the ConvRot W4A4 tensorwise linear on one MI355X.

Workload (the single MMDiT projection of the Qwen-Image MMDiT, per the
per-family shape table of the "Qwen-Image-Edit-2511-W4A8-ConvRot" card):
X bf16 [M, 3072] with M in {4096, 32} (image tokens and the small-token
case), N(0,1) with 15 outlier channels x30, W [3072, 3072] ~ N(0, 0.02)
prepared offline (rotated, quantized to INT4, tile-packed; untimed).

One step = the whole hot path for both token counts, inputs resident in HBM:
    rotate+quantize(X_4096) -> w4a4_gemm(4096)  ->  bf16 [4096, 3072]
    rotate+quantize(X_32)   -> w4a4_gemm(32)    ->  bf16 [32, 3072]
Every step uses a different copy of all buffers (inputs, weights, codes,
outputs; ~10 copies, over 2x the 256 MB last-level cache), so each step
reads cold HBM data.

The INT4 codes travel as fp6 E2M3 values and the GEMMs run on the fp6
matrix cores (exact: see gemm_f6.hip); `--cores int8` runs the int8-core
path instead (int4 tile-packed codes widened to bytes).

Metric: effective TOPS = sum 2*M*N*K / step time (the fused
rotate+quantize+W4 GEMM throughput), also given as % of the 5.0 POP/s dense
INT8 matrix peak. The roofline object reports the dominant kernel (the
M=4096 GEMM) against the dense peak of the matrix instruction it runs on
(fp6: 10.1 PFLOP/s; int8: 5.0 POP/s); its duration is the mean over K
back-to-back launches, timed with HIP events on the launch stream
(kernels_us.gemm_m4096_in_step: events around each launch inside the steps,
which also hold the launch gap). The M=4096 rotate+quantize (two launches)
is timed the same way for rq_m4096_GBps. The CPU baseline is the numpy oracle
running the same step on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--rot-group 256] [--cores fp6|int8]
                       [--workload c2|c1|c3|c4|c5|c2a8]
(--workload other than c2 prints that workload's throughput line instead;
see bench_workloads.py)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0       # MI355X dense INT8 matrix peak (5.0 POP/s)
FP6_PEAK_TOPS = 10100.0       # MI355X dense fp6 / fp4 matrix peak (10.1 PFLOP/s)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
M_BIG, M_SMALL, N, K = 4096, 32, 3072, 3072
ROT = 256          # ConvRot group size (--rot-group: 16, 64, 256 or 1024)
CORES = "fp6"      # matrix cores of the W4A4 GEMMs (--cores)
GEMM_SOURCES = {"fp6": ["gemm_f6.hip", "epilogue.h", "common.h", "kernels.h"],
                "int8": ["gemm_w4a4.hip", "epilogue.h", "common.h", "kernels.h"]}
TRAFFIC_PROFILE = {"fp6": "w4a4_f6_gemm_m4096_n3072_k3072_traffic.json",
                   "int8": "w4a4_gemm_m4096_n3072_k3072_traffic.json"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--rot-group", type=int, default=256, choices=(16, 64, 256, 1024),
                    help="ConvRot group size of the c2 line (256 is the configuration the metric is quoted on)")
    ap.add_argument("--cores", default="fp6", choices=("fp6", "int8"),
                    help="matrix cores of the W4A4 GEMMs: fp6 (E2M3 codes, default) or int8 (widened int4)")
    ap.add_argument("--workload", default="c2",
                    help="c2 (default: the headline line), or c1 / c3 / c4 / c5 / c2a8 / merge for the other workloads' "
                         "throughput lines (bench_workloads.py)")
    return ap.parse_args()


def source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "w4a8_rotated_quantized_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 counter summary, only if the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", TRAFFIC_PROFILE[CORES])
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_sha") != source_sha(GEMM_SOURCES[CORES]):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(budget_s):
    """The oracle (numpy) running the same step on the host, repeated until
    about budget_s seconds have passed."""
    import numpy as np
    import workloads as wl
    from oracle import linear as ol, gemm as og
    xb_big = wl.activation(2, 0, M_BIG, K, n_outliers=15, outlier_scale=30.0)
    xb_small = wl.activation(2, 2, M_SMALL, K, n_outliers=15, outlier_scale=30.0)
    wp = ol.prepare_w4a4(wl.weight(2, 1, N, K), ROT)
    try:
        import threadpoolctl
        np.ones((64, 64)) @ np.ones((64, 64))
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    reps, t0 = 0, time.perf_counter()
    while True:
        for xb in (xb_big, xb_small):
            r = ol.rotate_quantize(xb, ROT, "int4", "tensor")
            acc = og.int_gemm(r["values"], wp["values"])
            ol.epilogue_scalar(acc, r["scales"], "tensor", wp["scales"], "tensor")
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    ops = 2.0 * (M_BIG + M_SMALL) * N * K * reps
    return {"value": ops / el / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} full oracle step(s) (M=4096 and M=32, K=N=3072) in {el:.1f} s "
                      f"(numpy; elementwise stages single-threaded, BLAS threads={cores})"}


def setup(dev, nbytes_target=600e6):
    """Weights prepared offline (untimed) and enough buffer sets of every
    tensor that consecutive steps touch cold HBM data."""
    import numpy as np
    import torch
    import w4a8_rotated_quantized_amd as cr
    import workloads as wl

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    xb_big = wl.activation(2, 0, M_BIG, K, n_outliers=15, outlier_scale=30.0)
    xb_small = wl.activation(2, 2, M_SMALL, K, n_outliers=15, outlier_scale=30.0)
    wb = wl.weight(2, 1, N, K)
    w = bf16(wb)
    wc, ws, _, _ = cr.convrot_rotate_quantize(w, ROT, cr.Q.SYM_INT4, cr.GRAN.TENSOR)
    if CORES == "fp6":
        wp = cr.w4_pack_weights_f6(wc, N, K)
        code_shape = lambda m: ((m + 31) // 32, K // 64, 1536)   # noqa: E731
    else:
        wp, _, _, _ = cr.w4_pack_weights(wc, ws, N, K, cr.Q.SYM_INT4, cr.GRAN.TENSOR)
        code_shape = lambda m: ((m + 15) // 16, K // 64, 512)    # noqa: E731
    per_set = M_BIG * K * 2 + M_BIG * K // 2 + M_BIG * N * 2 + N * K // 2
    nsets = max(2, int(np.ceil(nbytes_target / per_set)))
    sets = []
    xbig0, xsmall0 = bf16(xb_big), bf16(xb_small)
    for _ in range(nsets):
        sets.append({
            "xb": xbig0.clone(), "xs": xsmall0.clone(), "wp": wp.clone(), "ws": ws.clone(),
            "cb": torch.empty(code_shape(M_BIG), dtype=torch.uint8, device=dev),
            "cs": torch.empty(code_shape(M_SMALL), dtype=torch.uint8, device=dev),
            "sb": torch.empty(1, dtype=torch.float32, device=dev),
            "ss": torch.empty(1, dtype=torch.float32, device=dev),
            "wsb": torch.empty(cr.convrot_rq_workspace_size(M_BIG, K, ROT, 0, 0), dtype=torch.uint8, device=dev),
            "wss": torch.empty(cr.convrot_rq_workspace_size(M_SMALL, K, ROT, 0, 0), dtype=torch.uint8, device=dev),
            "yb": torch.empty((M_BIG, N), dtype=torch.bfloat16, device=dev),
            "ys": torch.empty((M_SMALL, N), dtype=torch.bfloat16, device=dev),
        })
    return sets


def _layout(cr):
    return cr.LAYOUT.F6 if CORES == "fp6" else cr.LAYOUT.TILED


def rq_big(cr, s):
    cr.convrot_rotate_quantize(s["xb"], ROT, 0, 0, layout=_layout(cr), codes=s["cb"], scales=s["sb"],
                               workspace=s["wsb"])


def gemm_big(cr, s):
    cr.w4a4_gemm(s["cb"], s["sb"], 0, s["wp"], s["ws"], 0, M_BIG, N, K, out=s["yb"])


def rq_small(cr, s):
    cr.convrot_rotate_quantize(s["xs"], ROT, 0, 0, layout=_layout(cr), codes=s["cs"], scales=s["ss"],
                               workspace=s["wss"])


def gemm_small(cr, s):
    cr.w4a4_gemm(s["cs"], s["ss"], 0, s["wp"], s["ws"], 0, M_SMALL, N, K, out=s["ys"])


def main():
    global ROT, CORES
    args = parse()
    ROT = args.rot_group
    CORES = args.cores
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU part); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    if args.workload != "c2":
        import bench_workloads
        for name in args.workload.split(","):
            bench_workloads.run(name, args.steps, args.warmup, cores=args.cores)
        return

    import numpy as np
    import torch
    import w4a8_rotated_quantized_amd as cr

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sets = setup(dev)
    nsets = len(sets)

    ev = {}

    def step(i, record):
        s = sets[i % nsets]
        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            e[0].record(stream)
        rq_big(cr, s)
        if record:
            e[1].record(stream)
        gemm_big(cr, s)
        if record:
            e[2].record(stream)
        rq_small(cr, s)
        if record:
            e[3].record(stream)
        gemm_small(cr, s)
        if record:
            e[4].record(stream)
            ev.setdefault("e", []).append(e)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()

    # timed region 1: plain back-to-back steps (the headline number)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i, False)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # timed region 2: the same steps with events around every kernel call
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    parts = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in ev["e"]])
    t_rq_big, t_gemm_call, t_rq_small, t_gemm_small = (float(np.mean(parts[:, j])) for j in range(4))

    # timed region 3: the dominant kernel alone, launched back to back over the
    # buffer sets (the events of region 2 also hold each launch's gap)
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    for i in range(args.steps):
        gemm_big(cr, sets[i % nsets])
    g1.record(stream)
    torch.cuda.synchronize()
    t_gemm_big = g0.elapsed_time(g1) / args.steps
    # the same for the M=4096 rotate+quantize (its two launches)
    torch.cuda.synchronize()
    g0.record(stream)
    for i in range(args.steps):
        rq_big(cr, sets[i % nsets])
    g1.record(stream)
    torch.cuda.synchronize()
    t_rq_call, t_rq_big = t_rq_big, g0.elapsed_time(g1) / args.steps

    ops_step = 2.0 * (M_BIG + M_SMALL) * N * K
    eff_tops = ops_step / (ms_step * 1e-3) / 1e12
    gemm_tops = 2.0 * M_BIG * N * K / (t_gemm_big * 1e-3) / 1e12
    rq_bytes = M_BIG * K * 2 + M_BIG * K * (0.75 if CORES == "fp6" else 0.5) + 4   # bf16 in, codes (6 or 4 bits) out
    rq_gbs = rq_bytes / (t_rq_big * 1e-3) / 1e9
    cb = 0.75 if CORES == "fp6" else 0.5                      # bytes per code in the operand layout
    small_bytes = N * K * cb + M_SMALL * K * cb + M_SMALL * N * 2
    traffic = traffic_from_profile()
    peak = FP6_PEAK_TOPS if CORES == "fp6" else INT8_PEAK_TOPS

    line = {
        "metric": "effective TOPS of fused rotate+quant+W4 GEMM (% INT8 MFMA peak); GB/s",
        "value": round(eff_tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": f"MMDiT projection, W4A4 tensorwise ConvRot group {ROT}, "
                               "X bf16 [M, 3072] (M = 4096 and 32), W [3072, 3072]",
                   "M": [M_BIG, M_SMALL], "N": N, "K": K, "rot_group": ROT,
                   "matrix_cores": CORES, "buffer_sets": nsets},
        "pct_int8_peak": round(100.0 * eff_tops / INT8_PEAK_TOPS, 2),
        "kernels_us": {"rq_m4096": round(t_rq_big * 1e3, 2), "gemm_m4096": round(t_gemm_big * 1e3, 2),
                       "rq_m4096_in_step": round(t_rq_call * 1e3, 2),
                       "gemm_m4096_in_step": round(t_gemm_call * 1e3, 2),
                       "rq_m32": round(t_rq_small * 1e3, 2), "gemm_m32": round(t_gemm_small * 1e3, 2)},
        "rq_m4096_GBps": round(rq_gbs, 1),
        "rq_m4096_pct_hbm": round(100.0 * rq_gbs / HBM_PEAK_GBS, 1),
        "gemm_m4096_TOPS": round(gemm_tops, 1),
        "gemm_m32_GBps": round(small_bytes / (t_gemm_small * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / peak, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
