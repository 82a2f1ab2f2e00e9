"""Throughput of the other workloads (tiny layer, W4A8, mixed MMDiT block,
low-rank corrected g64), one JSON line each, for `bench.py --workload NAME`.

A step runs every rotate+quantize the workload needs (one per activation
tensor and format: layers that share an input share the pass) and every
GEMM, in order, on one stream, with inputs resident in HBM. Weights are
prepared offline (untimed). `value` = sum of 2*M*N*K over the layers / step
time. Per-kernel times come from HIP events around each launch in a second
pass; each GEMM is also reported as TOPS and, for M <= 64, as weight GB/s.
"""
import json
import sys
import time

INT8_PEAK_TOPS = 5000.0
HBM_PEAK_GBS = 8000.0


def _plan(w):
    """RQ passes (x_id, kind) and GEMMs for workload w. An activation that
    feeds both per-tensor INT4 and INT8 layers is quantized once, to both
    (convrot_rotate_quantize_dual)."""
    def kind_of(lin):
        return {"w4a4": "int4_tensor", "int8": "int8_tensor", "w4a8": "int8_row_f16", "a8w4": "int8_row",
                "w4a4_g64": ("u4_g64" if lin.unsigned_shift else "s4_g64")}[lin.fmt]
    kinds = {}
    for lin in w.linears:
        kinds.setdefault(lin.x_id, set()).add(kind_of(lin))
    rq, gemms = [], []
    for lin in w.linears:
        kind = kind_of(lin)
        if kind in ("int4_tensor", "int8_tensor") and {"int4_tensor", "int8_tensor"} <= kinds[lin.x_id]:
            kind = "dual_tensor"
        key = (lin.x_id, kind, lin.name if lin.fmt == "w4a4_g64" else "")
        if key not in rq:
            rq.append(key)
        gemms.append((lin, key))
    return rq, gemms


def run_merge(steps, warmup):
    """LoRA merge into a W4A8 weight (12288 x 3072, asym uint4 g16, ConvRot
    256) with a rank-64 delta: dequantize + delta, rotate + quantize again,
    pack; one JSON line with the time per merge and the bytes it moves."""
    import numpy as np
    import torch
    import w4a8_rotated_quantized_amd as cr
    import workloads as wl
    dev = torch.device("cuda:0")
    N, K, R = 12288, 3072, 64

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    w = wl.CONFIGS["c3"]()
    wb = bf16(wl.weight_bits(w, w.linears[0]))
    up, down = bf16(wl.weight(3, 700, N, R, std=0.05)), bf16(wl.weight(3, 701, R, K, std=0.05))
    codes, scales, zeros, _ = cr.convrot_rotate_quantize(wb, 256, cr.Q.ASYM_UINT4, cr.GRAN.ROW_GROUP, 16)
    merged = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    c2, s2, z2 = torch.empty_like(codes), torch.empty_like(scales), torch.empty_like(zeros)

    def step():
        cr.convrot_dequantize_weights(codes, scales, N, K, cr.Q.ASYM_UINT4, cr.GRAN.ROW_GROUP, 16, 256, zeros=zeros,
                                      delta_up=up, delta_down=down, out=merged)
        cr.convrot_rotate_quantize(merged, 256, cr.Q.ASYM_UINT4, cr.GRAN.ROW_GROUP, 16, codes=c2, scales=s2, zeros=z2)
        cr.w4_pack_weights(c2, s2, N, K, cr.Q.ASYM_UINT4, cr.GRAN.ROW_GROUP, 16, zeros=z2)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # bytes: codes + scales + zeros in, bf16 weight out and back in, new codes/scales/zeros, packed set
    q_bytes = N * K // 2 + N * K // 16 * 2 + N * K // 32
    moved = q_bytes + 2 * N * K + 2 * N * K + q_bytes + (N * K // 2 + N * K // 16 * 3 + 4 * N) + R * (N + K) * 2
    print(json.dumps({
        "metric": "LoRA merge into a quantized weight (dequantize + rank-64 delta + requantize + pack)",
        "value": round(ms, 4), "unit": "ms per merge", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "higher_is_better": False, "data": "synthetic",
        "config": {"workload": "W4A8 asym g16 weight 12288x3072, ConvRot 256, LoRA rank 64"},
        "GBps": round(moved / ms / 1e6, 1)}))


def run(name, steps, warmup, cores="fp6"):
    """cores: matrix cores of the W4A4 layers (per-tensor and 64-group),
    "fp6" (E2M3 fragments) or "int8" (tile-packed int4 widened to bytes)."""
    if name == "merge":
        return run_merge(steps, warmup)
    import numpy as np
    import torch
    import w4a8_rotated_quantized_amd as cr
    import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    w = wl.CONFIGS[name]()
    rq_plan, gemm_plan = _plan(w)
    f6 = cores == "fp6"

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    acts = {x: bf16(wl.act_bits(w, x)) for x in w.acts}
    # offline weight preparation and the low-rank factors
    prep = {}
    for lin in w.linears:
        N, K = lin.N, lin.K
        if lin.fmt in ("w4a4", "a8w4"):
            wc, ws, _, _ = cr.convrot_rotate_quantize(bf16(wl.weight_bits(w, lin)), 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR)
            if lin.fmt == "w4a4" and f6:
                prep[lin.name] = dict(w=cr.w4_pack_weights_f6(wc, N, K), ws=ws)
            else:
                prep[lin.name] = dict(w=cr.w4_pack_weights(wc, ws, N, K)[0], ws=ws)
        elif lin.fmt == "int8":
            wc, ws, _, _ = cr.convrot_rotate_quantize(bf16(wl.weight_bits(w, lin)), 256, cr.Q.SYM_INT8, cr.GRAN.TENSOR)
            prep[lin.name] = dict(w=wc, ws=ws)
        elif lin.fmt == "w4a8":
            wc, ws, wz, _ = cr.convrot_rotate_quantize(bf16(wl.weight_bits(w, lin)), 256, cr.Q.ASYM_UINT4,
                                                       cr.GRAN.ROW_GROUP, 16)
            p, ps, pz, _ = cr.w4_pack_weights(wc, ws, N, K, cr.Q.ASYM_UINT4, cr.GRAN.ROW_GROUP, 16, zeros=wz)
            prep[lin.name] = dict(w=p, ws=ps, wz=pz)
        else:
            l1, l2, r = wl.lowrank_bits(w, lin)
            wc, ws, _, _ = cr.convrot_rotate_quantize(bf16(r), 0, cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP, 64)
            p, ps, _, wsum = cr.w4_pack_weights(wc, ws, N, K, cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP, 64, want_wsum=True)
            if f6:
                p = cr.w4_pack_weights_f6(wc, N, K)
            prep[lin.name] = dict(w=p, ws=ps, wsum=wsum, l1=bf16(l1), l2=bf16(l2))
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    # RQ outputs, allocated once; per-tensor INT4 codes in the layout of the cores used
    lay4 = cr.LAYOUT.F6 if f6 else cr.LAYOUT.TILED

    def c4_shape(M, K):
        return ((M + 31) // 32, K // 64, 1536) if f6 else ((M + 15) // 16, K // 64, 512)

    rq_out = {}
    for key in rq_plan:
        x_id, kind, lname = key
        M, K = w.acts[x_id][0], w.acts[x_id][1]
        x = acts[x_id]
        if kind == "int4_tensor":
            o = dict(codes=torch.empty(c4_shape(M, K), dtype=torch.uint8, device=dev),
                     scales=torch.empty(1, dtype=torch.float32, device=dev),
                     ws=torch.empty(cr.convrot_rq_workspace_size(M, K, 256, 0, 0), dtype=torch.uint8, device=dev))
        elif kind == "int8_tensor":
            o = dict(codes=torch.empty((M, K), dtype=torch.int8, device=dev),
                     scales=torch.empty(1, dtype=torch.float32, device=dev),
                     ws=torch.empty(cr.convrot_rq_workspace_size(M, K, 256, 1, 0), dtype=torch.uint8, device=dev))
        elif kind == "dual_tensor":
            o = dict(codes=torch.empty(c4_shape(M, K), dtype=torch.uint8, device=dev),
                     scales=torch.empty(1, dtype=torch.float32, device=dev),
                     codes8=torch.empty((M, K), dtype=torch.int8, device=dev),
                     scales8=torch.empty(1, dtype=torch.float32, device=dev),
                     ws=torch.empty(cr.convrot_rq_workspace_size(M, K, 256, 0, 0), dtype=torch.uint8, device=dev))
        elif kind in ("int8_row", "int8_row_f16"):
            o = dict(codes=torch.empty((M, K), dtype=torch.float16 if kind == "int8_row_f16" else torch.int8,
                                       device=dev),
                     scales=torch.empty(M, dtype=torch.float32, device=dev), ws=None)
        else:
            o = dict(codes=torch.empty(c4_shape(M, K), dtype=torch.uint8, device=dev),
                     scales=torch.empty((M, K // 64), dtype=torch.float32, device=dev), ws=None,
                     la=torch.empty((M, 32), dtype=torch.bfloat16, device=dev))
        rq_out[key] = o
    outs = {lin.name: torch.empty((lin.M, lin.N), dtype=torch.bfloat16, device=dev) for lin in w.linears}

    def launch_rq(key):
        x_id, kind, lname = key
        o, x = rq_out[key], acts[x_id]
        if kind == "int4_tensor":
            cr.convrot_rotate_quantize(x, 256, cr.Q.SYM_INT4, cr.GRAN.TENSOR, layout=lay4,
                                       codes=o["codes"], scales=o["scales"], workspace=o["ws"])
        elif kind == "int8_tensor":
            cr.convrot_rotate_quantize(x, 256, cr.Q.SYM_INT8, cr.GRAN.TENSOR, codes=o["codes"],
                                       scales=o["scales"], workspace=o["ws"])
        elif kind == "dual_tensor":
            cr.convrot_rotate_quantize_dual(x, 256, layout4=lay4, codes4=o["codes"], scale4=o["scales"],
                                            codes8=o["codes8"], scale8=o["scales8"], workspace=o["ws"])
        elif kind in ("int8_row", "int8_row_f16"):
            cr.convrot_rotate_quantize(x, 256, cr.Q.SYM_INT8, cr.GRAN.ROW, codes=o["codes"], scales=o["scales"],
                                       layout=cr.LAYOUT.F16 if kind == "int8_row_f16" else cr.LAYOUT.NATURAL)
        else:
            lin = [l for l in w.linears if l.name == lname][0]
            uns = kind == "u4_g64"
            cr.convrot_rotate_quantize(x, 0, cr.Q.UNSIGNED_INT4_SHIFT if uns else cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP,
                                       64, shift=lin.unsigned_shift, lora_down=prep[lname]["l2"],
                                       layout=lay4, codes=o["codes"], scales=o["scales"],
                                       lora_act=o["la"])

    def launch_gemm(lin, key):
        o, p, y = rq_out[key], prep[lin.name], outs[lin.name]
        M, N, K = lin.M, lin.N, lin.K
        if lin.fmt == "w4a4":
            cr.w4a4_gemm(o["codes"], o["scales"], 0, p["w"], p["ws"], 0, M, N, K, out=y)
        elif lin.fmt == "a8w4":
            cr.w4a4_gemm(o["codes"], o["scales"], cr.GRAN.ROW, p["w"], p["ws"], 0, M, N, K, out=y,
                         a_layout=cr.LAYOUT.INT8)
        elif lin.fmt == "int8":
            a8, s8 = (o["codes8"], o["scales8"]) if "codes8" in o else (o["codes"], o["scales"])
            cr.int8_tensorwise_gemm(a8, s8, p["w"], p["ws"], M, N, K, out=y)
        elif lin.fmt == "w4a8":
            cr.w4a8_gemm(o["codes"], o["scales"], cr.GRAN.ROW, p["w"], p["ws"], p["wz"], M, N, K, out=y)
        else:
            cr.w4a4_gemm(o["codes"], o["scales"], 2, p["w"], p["ws"], 2, M, N, K,
                         a_unsigned=lin.unsigned_shift != 0.0, a_shift=lin.unsigned_shift, w_sum=p["wsum"],
                         lora_act=o["la"], lora_up=p["l1"], out=y)

    order = []   # (label, fn): every RQ right before the first GEMM that reads it
    done = set()
    for lin, key in gemm_plan:
        if key not in done:
            order.append((f"rq:{key[0]}:{key[1]}", lambda k=key: launch_rq(k)))
            done.add(key)
        order.append((f"gemm:{lin.name}", lambda l=lin, k=key: launch_gemm(l, k)))

    def step():
        for _, fn in order:
            fn()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps

    per = {lab: [] for lab, _ in order}
    for _ in range(max(3, steps // 2)):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
        ev[0].record(stream)
        for i, (_, fn) in enumerate(order):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        for i, (lab, _) in enumerate(order):
            per[lab].append(ev[i].elapsed_time(ev[i + 1]) * 1e3)
    kern = {lab: round(float(np.mean(v)), 2) for lab, v in per.items()}

    ops = sum(2.0 * l.M * l.N * l.K for l in w.linears)
    layers = {}
    for lin, _ in gemm_plan:
        us = kern[f"gemm:{lin.name}"]
        d = {"us": us, "TOPS": round(2.0 * lin.M * lin.N * lin.K / us / 1e6, 1)}
        if lin.M <= 64:
            wbytes = lin.N * lin.K // (1 if lin.fmt == "int8" else 2)
            d["weight_GBps"] = round(wbytes / us / 1e3, 1)
        layers[lin.name] = d
    rqs = {}
    for key in rq_plan:
        x_id, kind, _ = key
        M, K = w.acts[x_id][0], w.acts[x_id][1]
        us = kern[f"rq:{x_id}:{kind}"]
        code_b = 1.0 if kind.startswith("int8") else 0.5      # algorithmic: 8 or 4 bits per code
        out_b = M * K * code_b + (M * K if kind == "dual_tensor" else 0)
        rqs[f"{x_id}:{kind}"] = {"us": us, "GBps": round((M * K * 2 + out_b) / us / 1e3, 1)}
    dom = max(layers, key=lambda n: layers[n]["us"])
    eff = ops / (ms * 1e-3) / 1e12
    line = {
        "metric": "effective TOPS of fused rotate+quant+W4 GEMM (% INT8 MFMA peak); GB/s",
        "value": round(eff, 2), "unit": "TOPS", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4" if name not in ("c3", "c2a8") else "int8/int4", "data": "synthetic",
        "config": {"workload": w.name, "layers": len(w.linears), "total_GOP": round(ops / 1e9, 1),
                   "w4a4_matrix_cores": cores},
        "pct_int8_peak": round(100.0 * eff / INT8_PEAK_TOPS, 2),
        "gemm": layers, "rotate_quantize": rqs,
        "dominant_gemm": {"layer": dom, **layers[dom], "frac_int8_peak": round(layers[dom]["TOPS"] / INT8_PEAK_TOPS, 4)},
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(line))
