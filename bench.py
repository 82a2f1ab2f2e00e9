"""Benchmark of the ConvRot low-bit linear layer path on one MI355X.

Default workload: the mixed-precision MMDiT block (8192 image + 512 text
tokens, hidden 3072), the largest single-GPU configuration:
  * Q, K, MLP up (3072 -> 12288) and the post-GELU MLP down (12288 -> 3072)
    in W4A4 tensorwise ConvRot (INT4 x INT4),
  * V and attention output projections and the adaLN modulation linear
    (3072 -> 6 x 3072, 2 rows: one per sample of a batch of 2) in INT8
    tensorwise ConvRot,
for the image and the text stream: 14 linears, 1971.8 GOP per step. The
recipe follows the "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4" page
(intro: 480 INT4 and 359 INT8 layers; Measurements); the shapes follow the
per-family shape table of the "Qwen-Image-Edit-2511-W4A8-ConvRot" card. All
inputs are seeded synthetic tensors (workloads/): no model, dataset or
checkpoint. Weights are prepared offline (rotated, quantized, packed at 4
bits per INT4 code; untimed).

One step = every rotate+quantize pass and every GEMM of the block, the
image and text token streams on HIP streams of their own that meet between
the Q/K/V and the output projections (the joint attention) and at the end of
the step, inputs resident in HBM; two buffer sets (weights included,
~1.2 GB each, over 4x the 256 MB last-level cache) alternate, so every step
reads cold data. The W4A4 GEMMs expand their 4-bit weight tiles into fp6
E2M3 fragments in a workspace and run on the fp6 matrix cores (INT4 codes
are exact E2M3 values, the float32 sums exact); the INT8 layers run on the
int8 matrix cores; the 2-row modulation linears stream their weights.

Metric: effective TOPS = sum 2*M*N*K / step time (the fused
rotate+quant+W4 GEMM throughput), also as % of the 5.0 POP/s dense INT8
matrix peak; GB/s of every rotate+quantize pass (algorithmic bytes: bf16 in,
codes out at 4 or 8 bits per code). The roofline object reports the
dominant kernel (the GEMM kernel of the slowest layer) against the dense peak
of the matrix instruction it runs on, its duration the median over batches of back-to-back
launches timed with HIP events on the launch stream. Order on the GPU:
setup, a first window of W + K steps (reported as
ms_per_step_first_window), the per-call, dominant-kernel, clock and
one-stream measurements, then the headline window of W untimed and K timed
steps. The same line carries
the single MMDiT projection (M = 4096 and M = 32) as "c2". The CPU baseline
is the numpy oracle running a bounded sample of the same block on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--cores fp6|int8]
                       [--workload c4|c2|c1|c3|c5|c2a8|merge]
(--workload other than c4 prints that workload's line; see bench_workloads.py)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench_workloads as bw  # noqa: E402

GEMM_SOURCES = {"fp6": ["gemm_f6.hip", "epilogue.h", "common.h", "kernels.h"],
                "int8": ["gemm_w4a4.hip", "epilogue.h", "common.h", "kernels.h"]}
TRAFFIC_PROFILE = {"fp6": "c4_img_mlp_gemm_f6_traffic.json", "int8": "c4_img_mlp_gemm_int8_traffic.json"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cores", default="fp6", choices=("fp6", "int8"),
                    help="matrix cores of the W4A4 GEMMs above 64 tokens: fp6 (default) or int8")
    ap.add_argument("--workload", default="c4",
                    help="c4 (default: the headline line), or c1 / c2 / c3 / c5 / c2a8 / merge for the other "
                         "workloads' throughput lines (bench_workloads.py)")
    ap.add_argument("--rot-group", type=int, default=256, choices=(16, 64, 256, 1024),
                    help="ConvRot group size of the W4A4 / INT8 tensorwise layers of --workload c1 / c2 / c4")
    return ap.parse_args()


def source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "w4a8_rotated_quantized_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(cores, layer):
    """HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 counter summary, only if it covers this layer and the kernel
    source is unchanged."""
    p = os.path.join(ROOT, "profiles", TRAFFIC_PROFILE[cores])
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_sha") != source_sha(GEMM_SOURCES[cores]) or d.get("layer") != layer:
        return None
    return d.get("hbm_bytes_per_launch")


def stream_copy_gbs():
    """Bytes moved per second (read + write) by a device-to-device copy of
    1 GiB, median of 5 (after 2 untimed), HIP events on the launch stream:
    the box's streaming bandwidth that the quantizers are also reported
    against."""
    import torch
    n = 1 << 29                                   # bf16 elements: 1 GiB
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    s = torch.cuda.current_stream()
    ts = []
    for i in range(7):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        b.copy_(a)
        e1.record(s)
        e1.synchronize()
        if i >= 2:
            ts.append(e0.elapsed_time(e1))
    ts.sort()
    del a, b
    torch.cuda.empty_cache()
    return 2.0 * n * 2 / (ts[len(ts) // 2] * 1e-3) / 1e9


def _blas_threads():
    import numpy as np
    try:
        import threadpoolctl
        np.ones((64, 64)) @ np.ones((64, 64))
        info = threadpoolctl.threadpool_info()
        return max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline_workload(name, budget_s, rot=256):
    """The oracle (numpy) on a bounded sample of workload `name`, for the
    side lines: every linear on the first 512 rows of its input and its first
    1536 output channels, in the linear's own format (W4A4 tensorwise, INT8,
    W4A8 asymmetric g16 against per-token INT8, 8-bit activations against
    W4A4 weights, or the low-rank corrected 64-group format). Weights (and
    the low-rank split) prepared once, untimed."""
    import numpy as np  # noqa: F401
    import workloads as wl
    from oracle import linear as ol, gemm as og
    w = wl.CONFIGS[name]()
    NS, MR = 1536, 512
    jobs = []
    for lin in w.linears:
        rows = min(MR, w.acts[lin.x_id][0])
        x = wl.act_bits(w, lin.x_id, rows=rows)
        ns = min(NS, lin.N)
        r = rot                                 # the runner's rotation of the tensorwise formats
        if lin.fmt == "w4a4":
            wp = ol.prepare_w4a4(wl.weight_bits(w, lin, rows=ns), r)
            jobs.append((lambda x=x, wp=wp, r=r: ol.w4a4_linear(x, None, r, wprep=wp), rows, ns, lin.K))
        elif lin.fmt == "int8":
            wq = ol.rotate_quantize(wl.weight_bits(w, lin, rows=ns), r, "int8", "tensor")

            def f(x=x, wq=wq, r=r):
                xa = ol.rotate_quantize(x, r, "int8", "tensor")
                acc = og.int_gemm(xa["values"], wq["values"])
                return ol.epilogue_scalar(acc, xa["scales"], "tensor", wq["scales"], "tensor")
            jobs.append((f, rows, ns, lin.K))
        elif lin.fmt == "a8w4":
            wp = ol.prepare_w4a4(wl.weight_bits(w, lin, rows=ns), r)
            jobs.append((lambda x=x, wp=wp, r=r: ol.a8w4_linear(x, None, r, a_gran="row", wprep=wp), rows, ns, lin.K))
        elif lin.fmt == "w4a8":
            wp = ol.prepare_w4a8(wl.weight_bits(w, lin, rows=ns), 256, 16)
            jobs.append((lambda x=x, wp=wp: ol.w4a8_linear(x, None, 256, 16, wprep=wp), rows, ns, lin.K))
        else:                                   # low-rank corrected, 64-group scales, rotation off
            l1, l2, res = wl.lowrank_bits(w, lin)
            wp = ol.prepare_w4a4(res[:ns], 0, "row_group", 64)
            jobs.append((lambda x=x, wp=wp, l1=l1[:ns], l2=l2, sh=lin.unsigned_shift:
                         ol.w4a4_linear(x, None, 0, "row_group", "row_group", 64, sh, l1, l2, wprep=wp),
                         rows, ns, lin.K))
    cores = _blas_threads()
    ops1 = sum(2.0 * rows * ns * K for _, rows, ns, K in jobs)
    reps, t0 = 0, time.perf_counter()
    while True:
        for fn, _, _, _ in jobs:
            fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": ops1 * reps / el / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} pass(es) of the workload's {len(jobs)} linear(s) on the first {MR} rows of each "
                      f"input and the first {NS} output channels of each weight ({ops1 / 1e9:.1f} GOP each) in "
                      f"{el:.1f} s (numpy; rotation and quantization single-threaded, integer products as "
                      f"float64 BLAS, BLAS threads={cores})"}


def cpu_baseline(budget_s):
    """The oracle (numpy) running a bounded sample of the block on the host:
    all 14 layers on the first 512 rows of every activation tensor (all of
    the text and modulation tensors) and the first 1536 output channels of
    every weight. Weights prepared once, untimed."""
    import numpy as np
    import workloads as wl
    from oracle import linear as ol, gemm as og
    w = wl.CONFIGS["c4"]()
    NS = 1536
    rows = {x: min(512, w.acts[x][0]) for x in w.acts}
    acts = {x: wl.act_bits(w, x, rows=rows[x]) for x in w.acts}
    wq = {}
    for lin in w.linears:
        qt = "int4" if lin.fmt == "w4a4" else "int8"
        wq[lin.name] = ol.rotate_quantize(wl.weight_bits(w, lin, rows=NS), 256, qt, "tensor")
    try:
        import threadpoolctl
        np.ones((64, 64)) @ np.ones((64, 64))
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    ops1 = sum(2.0 * rows[l.x_id] * min(l.N, NS) * l.K for l in w.linears)
    reps, t0 = 0, time.perf_counter()
    while True:
        rq = {}
        for lin in w.linears:
            qt = "int4" if lin.fmt == "w4a4" else "int8"
            key = (lin.x_id, qt)
            if key not in rq:
                rq[key] = ol.rotate_quantize(acts[lin.x_id], 256, qt, "tensor")
            xa, wp = rq[key], wq[lin.name]
            acc = og.int_gemm(xa["values"], wp["values"])
            ol.epilogue_scalar(acc, xa["scales"], "tensor", wp["scales"], "tensor")
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": ops1 * reps / el / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} pass(es) of the block's 14 layers on the first 512 image tokens, all 512 text "
                      f"tokens and both modulation rows, first {NS} output channels of each weight "
                      f"({ops1 / 1e9:.1f} GOP each) in {el:.1f} s (numpy; "
                      f"rotation and quantization single-threaded, integer GEMM as float64 BLAS, "
                      f"BLAS threads={cores})"}


def c2_line(steps, warmup, cores):
    # one stream: this short step runs slower with its two chains on two
    # streams (both figures are reported)
    r = bw.Runner("c2", cores)
    ms = r.time_steps(steps, warmup)
    ms_chains = r.time_steps(steps, warmup, schedule="chains")
    kern = r.per_call(max(3, steps // 2))
    big = [l for l in r.w.linears if l.M == 4096][0]
    t_gemm = r.gemm_kernel_median(big)
    out = {"workload": r.w.name, "value": round(r.ops() / (ms * 1e-3) / 1e12, 2), "unit": "TOPS",
           "ms_per_step": round(ms, 5), "ms_per_step_two_streams": round(ms_chains, 5),
           "schedule": "one stream",
           "kernels_us": {k.replace(":x", ":m").replace(":int4_tensor", ""): round(v, 2) for k, v in kern.items()},
           "gemm_m4096_kernel_us": round(t_gemm, 2),
           "gemm_m4096_TOPS": round(2.0 * big.M * big.N * big.K / t_gemm / 1e6, 1)}
    for lin in r.w.linears:
        us = kern[f"gemm:{lin.name}"]
        out[f"gemm_m{lin.M}_GBps"] = round(bw.gemm_bytes(lin) / us / 1e3, 1)
    for key in r.rq_plan:
        M, K = r.w.acts[key[0]][0], r.w.acts[key[0]][1]
        us = kern[f"rq:{key[0]}:{key[1]}"]
        out[f"rq_m{M}_GBps"] = round(bw.rq_bytes(M, K, key[1]) / us / 1e3, 1)
    del r
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU part); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if args.workload != "c4":
        for name in args.workload.split(","):
            extra = None
            if not args.no_cpu and name != "merge":
                def extra(line, name=name):
                    line["cpu_baseline"] = cpu_baseline_workload(name, args.cpu_seconds, args.rot_group)
            bw.run(name, args.steps, args.warmup, cores=args.cores, rot=args.rot_group, extra=extra)
        return

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)

    # both token streams concurrently; each stream's Q and K projections (one
    # input, one shape) as one call on their weights side by side
    r = bw.Runner("c4", args.cores, rot=args.rot_group, schedule="chains", fuse=True)
    # The first window right after setup is reported on its own: its first
    # step carries one-time initialisation and the next ~15 steps run 5-20%
    # slower than the sustained rate while the GPU ramps up under load. The
    # per-call, dominant-kernel, clock and one-stream measurements come next,
    # and the headline window (W untimed + K timed steps) after them.
    ms_first = r.time_steps(args.steps, args.warmup)
    chains = list(r.chains)
    kern = r.per_call(max(3, args.steps // 2))
    layers = {}
    for lin, _ in r.gemm_plan:
        us = kern[f"gemm:{lin.name}"]
        layers[lin.name] = {"us": round(us, 2), "TOPS": round(2.0 * lin.M * lin.N * lin.K / us / 1e6, 1),
                            "GBps": round(bw.gemm_bytes(lin) / us / 1e3, 1)}
    copy_gbs = stream_copy_gbs()
    rqs = {}
    for key in r.rq_plan:
        M, K = r.w.acts[key[0]][0], r.w.acts[key[0]][1]
        us = kern[f"rq:{key[0]}:{key[1]}"]
        gbs = bw.rq_bytes(M, K, key[1]) / us / 1e3
        rqs[f"{key[0]}:{key[1]}"] = {"us": round(us, 2), "GBps": round(gbs, 1),
                                     "pct_hbm": round(100.0 * gbs / bw.HBM_PEAK_GBS, 1),
                                     "pct_stream_copy": round(100.0 * gbs / copy_gbs, 1)}
    # dominant kernel: the GEMM kernel of the slowest layer, alone, back to back (median of 7 batches)
    dom = max(layers, key=lambda n: layers[n]["us"])
    dlin = [l for l in r.w.linears if l.name == dom][0]
    t_dom = r.gemm_kernel_median(dlin)
    dom_fn = r.gemm_kernel_fn(dlin)
    clock = {"steps": r.shader_clock(r.step, 200),
             "dominant_kernel": r.shader_clock(lambda i: dom_fn(i % r.nsets), max(200, int(2e5 / t_dom))),
             "nominal": 2400,
             "source": "amdsmi current_gfxclks of every XCD, read every ~2 ms from a host thread while "
                       "untimed whole steps (then the dominant kernel alone) keep the GPU busy"}
    ms_serial = r.time_steps(args.steps, args.warmup, schedule="serial")
    ms = r.time_steps(args.steps, args.warmup)
    eff = r.ops() / (ms * 1e-3) / 1e12
    on_f6 = dlin.fmt == "w4a4" and args.cores == "fp6" and dlin.M > bw.SKINNY_M
    peak = bw.FP6_PEAK_TOPS if on_f6 else bw.INT8_PEAK_TOPS
    achieved = 2.0 * dlin.M * dlin.N * dlin.K / t_dom / 1e6
    ops = r.ops()
    nsets = r.nsets
    name = r.w.name
    del r
    torch.cuda.empty_cache()

    line = {
        "metric": "effective TOPS of fused rotate+quant+W4 GEMM (% INT8 MFMA peak); GB/s",
        "value": round(eff, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_one_stream": round(ms_serial, 5),
        "ms_per_step_first_window": round(ms_first, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int4 x int4 (W4A4 layers: codes as fp6 E2M3 on the fp6 matrix cores, exact float32 sums) and "
                  "int8 x int8 (INT8 layers: int8 matrix cores, int32 sums)" if args.cores == "fp6" else
                  "int4 x int4 (widened to int8 on the int8 matrix cores) and int8 x int8, int32 sums"),
        "data": "synthetic",
        "config": {"workload": name, "layers": 14, "total_GOP": round(ops / 1e9, 1),
                   "tokens": {"image": 8192, "text": 512, "modulation_rows": 2}, "hidden": 3072,
                   "convrot_group": args.rot_group,
                   "w4a4_layers": "q, k, mlp_up, mlp_down (image and text)",
                   "fused_calls": "q and k of each stream in one GEMM call (weights side by side, N = 6144, "
                                  "each with its own per-tensor scale as per-channel scales): 12 GEMM calls",
                   "int8_layers": "v, out, mod (image and text)",
                   "w4a4_weights": "tile-packed INT4, 2 per byte (expanded per call into fp6 fragments)",
                   "w4a4_matrix_cores": args.cores, "buffer_sets": nsets,
                   "schedule": f"token streams {' and '.join(chains)} on streams of their own, meeting "
                               f"between the Q/K/V and the output projections (joint attention) and at "
                               f"the end of every step"},
        "pct_int8_peak": round(100.0 * eff / bw.INT8_PEAK_TOPS, 2),
        "gemm": layers,
        "rotate_quantize": rqs,
        "stream_copy_GBps": round(copy_gbs, 1),
        "shader_clock_MHz": clock,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic_from_profile(args.cores, dom),
                     "kernel": ("gemm_f6_kernel" if on_f6 else "int8-core GEMM") + f" of {dom} "
                               f"({dlin.M}x{dlin.N}x{dlin.K})", "kernel_us": round(t_dom, 2)},
    }
    line["c2"] = c2_line(args.steps, args.warmup, args.cores)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
