"""Workload runner of the benchmark: builds a workload's layers on the GPU
path (weights prepared offline, untimed), keeps several cold buffer sets, and
times whole steps and single calls with HIP events on the launch stream.

A step runs every rotate+quantize the workload needs (one per activation
tensor and code format: layers that share an input share the pass; an input
that feeds both INT4 and INT8 layers is quantized once to both) and every
GEMM, with inputs resident in HBM. With the "chains" schedule each chain of
layers (an independent token stream: the image and text tokens of an MMDiT
block) runs in order on a stream of its own; the chains meet between phases
(the joint attention between the Q/K/V projections and the output
projections) and before the step ends, and the next step starts after the
whole of it. The "serial" schedule
(step_serial) runs the same calls in order on one stream. Each step uses the
next buffer set (inputs, weights, codes, workspaces, outputs), so consecutive
steps read data the previous step did not touch.

Formats on the measured path:
  * W4A4 weights are stored tile-packed at 4 bits per code (w4_pack_weights).
    With more than 64 tokens the activation codes are fp6 E2M3 fragments and
    each GEMM call first expands the layer's weight tiles into fp6 fragments
    in a workspace, then runs the fp6 matrix-core GEMM ("fp6" cores); with
    64 tokens or fewer (and with cores="int8") the codes are tile-packed int4
    and the int8 matrix cores read the 4-bit tiles directly.
  * INT8 layers: int8 codes and weights on the int8 matrix cores.
  * W4A8: int8 activation codes carried as fp16 values, asymmetric uint4 g16
    weights, exact group partials on the fp16 matrix cores.
"""
import json
import sys
import time

INT8_PEAK_TOPS = 5000.0       # MI355X dense INT8 matrix peak (5.0 POP/s)
FP6_PEAK_TOPS = 10100.0       # MI355X dense fp6 / fp4 matrix peak (10.1 PFLOP/s)
FP16_PEAK_TOPS = 2500.0       # MI355X dense fp16 / bf16 matrix peak (2.5 PFLOP/s)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
# float32 FMAs on the vector ALUs without packed math: 256 CUs x 4 SIMDs x 16
# lanes x 2 flops x 2.4 GHz (the 157.3 TFLOP/s figure counts packed FMAs)
VALU_FP32_TFLOPS = 78.6

SKINNY_M = 64                 # token counts up to this take the weight-streaming int8-core kernels


def _kind_of(lin, cores):
    if lin.fmt == "w4a4":
        return "int4_tensor"
    if lin.fmt == "int8":
        return "int8_tensor"
    if lin.fmt == "w4a8":
        return "int8_row_f16"
    if lin.fmt == "a8w4":
        return "int8_row"
    return "u4_g64" if lin.unsigned_shift else "s4_g64"


def fuse_shared_inputs(w):
    """The workload with every run of W4A4 tensorwise layers that read the
    same input with the same token count, depth, chain and phase (an MMDiT
    block's Q and K projections) merged into one layer: one GEMM call on
    their weights side by side along N, each part keeping its own per-tensor
    weight scale (carried as per-channel scales). Every output element is
    computed by the same arithmetic as in the separate calls."""
    import workloads as wl
    out = wl.Workload(w.config_id, w.name, acts=dict(w.acts))
    lins = list(w.linears)
    i = 0
    while i < len(lins):
        a = lins[i]
        grp = [a]
        while (a.fmt == "w4a4" and i + len(grp) < len(lins)):
            b = lins[i + len(grp)]
            if (b.fmt, b.x_id, b.M, b.K, b.chain, b.phase, b.rot) != (a.fmt, a.x_id, a.M, a.K, a.chain, a.phase, a.rot):
                break
            grp.append(b)
        if len(grp) == 1:
            out.linears.append(a)
        else:
            out.linears.append(wl.LinearSpec("+".join(l.name for l in grp), "w4a4", a.M, sum(l.N for l in grp), a.K,
                                             a.x_id, rot=a.rot, chain=a.chain, phase=a.phase, parts=tuple(grp)))
        i += len(grp)
    return out


def plan(w, cores="fp6"):
    """RQ passes (x_id, kind, layer) and GEMMs (lin, rq key) of workload w."""
    kinds = {}
    for lin in w.linears:
        kinds.setdefault(lin.x_id, set()).add(_kind_of(lin, cores))
    rq, gemms = [], []
    for lin in w.linears:
        kind = _kind_of(lin, cores)
        if kind in ("int4_tensor", "int8_tensor") and {"int4_tensor", "int8_tensor"} <= kinds[lin.x_id]:
            kind = "dual_tensor"
        key = (lin.x_id, kind, lin.name if lin.fmt == "w4a4_g64" else "")
        if key not in rq:
            rq.append(key)
        gemms.append((lin, key))
    return rq, gemms


def rq_bytes(M, K, kind):
    """Algorithmic bytes of one rotate+quantize pass: bf16 in, codes out at
    their bit width (4 for INT4, 8 for INT8, both for the dual pass), plus
    the scales."""
    codes = {"int4_tensor": 0.5, "s4_g64": 0.5, "u4_g64": 0.5, "int8_tensor": 1.0, "int8_row": 1.0,
             "int8_row_f16": 1.0, "dual_tensor": 1.5}[kind]
    scales = {"int4_tensor": 4, "int8_tensor": 4, "dual_tensor": 8, "int8_row": 4 * M, "int8_row_f16": 4 * M,
              "s4_g64": 4 * M * K // 64, "u4_g64": 4 * M * K // 64}[kind]
    return 2 * M * K + codes * M * K + scales


def gemm_bytes(lin):
    """Algorithmic bytes of one GEMM: activation codes and weights at their
    bit width (INT4 0.5 B, INT8 1 B per code; W4A8 also fp16 scales and uint4
    zero points per 16 weights; 64-group scales as float32) and the bf16 output."""
    M, N, K = lin.M, lin.N, lin.K
    if lin.fmt == "w4a4":
        return 0.5 * M * K + 0.5 * N * K + 2 * M * N
    if lin.fmt == "int8":
        return M * K + N * K + 2 * M * N
    if lin.fmt == "w4a8":
        return M * K + N * K * (0.5 + 2.5 / 16) + 2 * M * N
    if lin.fmt == "a8w4":
        return M * K + 0.5 * N * K + 2 * M * N
    return 0.5 * M * K + 0.5 * N * K + 4 * (M + N) * K // 64 + 2 * M * N + 2 * lin.rank * (M + N)


def gemm_roofline(lin, us, cores="fp6"):
    """Roofline of one GEMM kernel of `us` microseconds against what bounds it:
    the weight bytes for M <= SKINNY_M, the vector ALUs for the per-group
    scaling of W4A8 (one float32 FMA per output and 16-group) and of the
    64-group format (per 64-group), else the matrix cores of its operand
    type (fp6 for W4A4 codes carried as E2M3, int8 otherwise)."""
    M, N, K = lin.M, lin.N, lin.K
    if M <= SKINNY_M:
        bound, unit, peak, work = "hbm", "GB/s", HBM_PEAK_GBS, gemm_bytes(lin)
        achieved = work / us / 1e3
    elif lin.fmt in ("w4a8", "w4a4_g64"):
        group = 16 if lin.fmt == "w4a8" else 64
        bound, unit, peak = "alu", "TFLOP/s", VALU_FP32_TFLOPS
        work = 2.0 * M * N * (K // group)
        achieved = work / us / 1e6
    else:
        on_f6 = lin.fmt == "w4a4" and cores == "fp6"
        bound, unit, peak = "mfma", "TFLOP/s", (FP6_PEAK_TOPS if on_f6 else INT8_PEAK_TOPS)
        work = 2.0 * M * N * K
        achieved = work / us / 1e6
    return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None, "kernel_us": round(us, 2)}


class Runner:
    """One workload on the GPU path with `nsets` cold buffer sets."""

    def __init__(self, name, cores="fp6", nsets=2, rot=256, workload=None, schedule="serial", fuse=False):
        import numpy as np
        import torch
        import w4a8_rotated_quantized_amd as cr
        import workloads as wl
        self.np, self.torch, self.cr = np, torch, cr
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.stream = torch.cuda.current_stream()
        self.w = workload if workload is not None else wl.CONFIGS[name]()
        w_def = self.w                 # the workload as defined (weights are drawn per defined linear)
        if fuse:
            self.w = fuse_shared_inputs(self.w)
        self.cores = cores
        self.rot = rot
        self.nsets = nsets
        dev = self.dev
        w = self.w
        self.rq_plan, self.gemm_plan = plan(w, cores)
        self.chains = list(dict.fromkeys(lin.chain for lin in w.linears))

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        t0 = time.time()
        acts = {x: bf16(wl.act_bits(w, x)) for x in w.acts}
        # offline weight preparation (untimed): rotate, quantize, pack
        prep = {}
        for lin in w.linears:
            N, K = lin.N, lin.K
            if lin.parts:
                # each part rotated, quantized (per-tensor scale) and packed on
                # its own; tiles and scales side by side along N
                tiles, scales = [], []
                for part in lin.parts:
                    wc, ws, _, _ = cr.convrot_rotate_quantize(bf16(wl.weight_bits(w_def, part)), rot, cr.Q.SYM_INT4,
                                                              cr.GRAN.TENSOR)
                    tiles.append(cr.w4_pack_weights(wc, ws, part.N, K)[0])
                    scales.append(ws.expand(part.N))
                prep[lin.name] = dict(w=torch.cat(tiles), ws=torch.cat(scales).contiguous(), w_gran=cr.GRAN.ROW)
            elif lin.fmt in ("w4a4", "a8w4"):
                wc, ws, _, _ = cr.convrot_rotate_quantize(bf16(wl.weight_bits(w_def, lin)), rot, cr.Q.SYM_INT4,
                                                          cr.GRAN.TENSOR)
                prep[lin.name] = dict(w=cr.w4_pack_weights(wc, ws, N, K)[0], ws=ws)
            elif lin.fmt == "int8":
                wc, ws, _, _ = cr.convrot_rotate_quantize(bf16(wl.weight_bits(w_def, lin)), rot, cr.Q.SYM_INT8,
                                                          cr.GRAN.TENSOR)
                prep[lin.name] = dict(w=wc, ws=ws)
            elif lin.fmt == "w4a8":
                wc, ws, wz, _ = cr.convrot_rotate_quantize(bf16(wl.weight_bits(w_def, lin)), 256, cr.Q.ASYM_UINT4,
                                                           cr.GRAN.ROW_GROUP, 16)
                p, ps, pz, _ = cr.w4_pack_weights(wc, ws, N, K, cr.Q.ASYM_UINT4, cr.GRAN.ROW_GROUP, 16, zeros=wz)
                prep[lin.name] = dict(w=p, ws=ps, wz=pz)
            else:
                l1, l2, r = wl.lowrank_bits(w_def, lin)
                wc, ws, _, _ = cr.convrot_rotate_quantize(bf16(r), 0, cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP, 64)
                p, ps, _, wsum = cr.w4_pack_weights(wc, ws, N, K, cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP, 64,
                                                    want_wsum=True)
                prep[lin.name] = dict(w=p, ws=ps, wsum=wsum, l1=cr.w4_pack_lora_up(bf16(l1)), l2=bf16(l2))
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0

        def f6_codes(M):
            return self.f6 and M > SKINNY_M
        self.f6 = cores == "fp6"
        self.f6_codes = f6_codes

        def c4_shape(M, K):
            return ((M + 31) // 32, K // 64, 1536) if f6_codes(M) else ((M + 15) // 16, K // 64, 512)

        ws_bytes = max([cr.w4a4_gemm_workspace_size(l.N, l.K, cr.LAYOUT.F6, cr.LAYOUT.TILED)
                        for l in w.linears if l.fmt in ("w4a4", "w4a4_g64")] + [16])
        self.sets = []
        for si in range(nsets):
            st = {"acts": {k: (v if si == 0 else v.clone()) for k, v in acts.items()},
                  "prep": {k: {kk: (vv if si == 0 or not hasattr(vv, "clone") else vv.clone()) for kk, vv in d.items()}
                           for k, d in prep.items()},
                  "rq": {}}
            # one GEMM workspace (weight expansion target) per chain: chains may run concurrently
            st["gws_c"] = {c: torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for c in self.chains}
            st["gws"] = st["gws_c"][self.chains[0]]
            for key in self.rq_plan:
                x_id, kind, lname = key
                M, K = w.acts[x_id][0], w.acts[x_id][1]
                rq_ws = lambda q: torch.empty(max(16, cr.convrot_rq_workspace_size(M, K, rot, q, 0)),  # noqa: E731
                                              dtype=torch.uint8, device=dev)
                if kind == "int4_tensor":
                    o = dict(codes=torch.empty(c4_shape(M, K), dtype=torch.uint8, device=dev),
                             scales=torch.empty(1, dtype=torch.float32, device=dev), ws=rq_ws(0))
                elif kind == "int8_tensor":
                    o = dict(codes=torch.empty((M, K), dtype=torch.int8, device=dev),
                             scales=torch.empty(1, dtype=torch.float32, device=dev), ws=rq_ws(1))
                elif kind == "dual_tensor":
                    o = dict(codes=torch.empty(c4_shape(M, K), dtype=torch.uint8, device=dev),
                             scales=torch.empty(1, dtype=torch.float32, device=dev),
                             codes8=torch.empty((M, K), dtype=torch.int8, device=dev),
                             scales8=torch.empty(1, dtype=torch.float32, device=dev), ws=rq_ws(0))
                elif kind in ("int8_row", "int8_row_f16"):
                    o = dict(codes=torch.empty((M, K), dtype=torch.float16 if kind == "int8_row_f16" else torch.int8,
                                               device=dev),
                             scales=torch.empty(M, dtype=torch.float32, device=dev), ws=None)
                else:
                    o = dict(codes=torch.empty(c4_shape(M, K), dtype=torch.uint8, device=dev),
                             scales=torch.empty((M, K // 64), dtype=torch.float32, device=dev), ws=None,
                             la=torch.empty((M, 32), dtype=torch.bfloat16, device=dev))
                st["rq"][key] = o
            st["out"] = {lin.name: torch.empty((lin.M, lin.N), dtype=torch.bfloat16, device=dev) for lin in w.linears}
            self.sets.append(st)
        del acts, prep
        torch.cuda.synchronize()

        self.order = []          # (label, fn(set index)): every RQ right before the first GEMM that reads it
        done = set()
        for lin, key in self.gemm_plan:
            if key not in done:
                self.order.append((f"rq:{key[0]}:{key[1]}", lambda si, k=key: self.launch_rq(si, k)))
                done.add(key)
            self.order.append((f"gemm:{lin.name}", lambda si, l=lin, k=key: self.launch_gemm(si, l, k)))

        # Chains schedule of a step: every chain (independent token stream)
        # in its order on a stream of its own, all chains meeting between
        # phases (corder[phase][chain] = launches).
        self.phases = sorted({lin.phase for lin in w.linears})
        self.corder = {ph: {c: [] for c in self.chains} for ph in self.phases}
        for lab, fn in self.order:
            lin = self._lin_of(lab)
            self.corder[lin.phase][lin.chain].append(fn)
        self.side = [torch.cuda.Stream() for _ in range(len(self.chains) - 1)]
        self.schedule = schedule if len(self.chains) > 1 else "serial"

    # ------------------------------------------------------------------
    def _lin_of(self, label):
        """the layer a launch label belongs to (an RQ: the first layer reading its input)"""
        kind, _, rest = label.partition(":")
        if kind == "gemm":
            return [l for l in self.w.linears if l.name == rest][0]
        x_id = rest.split(":")[0]
        return [l for l in self.w.linears if l.x_id == x_id][0]

    def _lay4(self, M):
        return self.cr.LAYOUT.F6 if self.f6_codes(M) else self.cr.LAYOUT.TILED

    def launch_rq(self, si, key):
        cr = self.cr
        x_id, kind, lname = key
        st = self.sets[si]
        o, x = st["rq"][key], st["acts"][x_id]
        M = x.shape[0]
        if kind == "int4_tensor":
            cr.convrot_rotate_quantize(x, self.rot, cr.Q.SYM_INT4, cr.GRAN.TENSOR, layout=self._lay4(M),
                                       codes=o["codes"], scales=o["scales"], workspace=o["ws"])
        elif kind == "int8_tensor":
            cr.convrot_rotate_quantize(x, self.rot, cr.Q.SYM_INT8, cr.GRAN.TENSOR, codes=o["codes"],
                                       scales=o["scales"], workspace=o["ws"])
        elif kind == "dual_tensor":
            cr.convrot_rotate_quantize_dual(x, self.rot, layout4=self._lay4(M), codes4=o["codes"],
                                            scale4=o["scales"], codes8=o["codes8"], scale8=o["scales8"],
                                            workspace=o["ws"])
        elif kind in ("int8_row", "int8_row_f16"):
            cr.convrot_rotate_quantize(x, 256, cr.Q.SYM_INT8, cr.GRAN.ROW, codes=o["codes"], scales=o["scales"],
                                       layout=cr.LAYOUT.F16 if kind == "int8_row_f16" else cr.LAYOUT.NATURAL)
        else:
            lin = [l for l in self.w.linears if l.name == lname][0]
            uns = kind == "u4_g64"
            cr.convrot_rotate_quantize(x, 0, cr.Q.UNSIGNED_INT4_SHIFT if uns else cr.Q.SYM_INT4, cr.GRAN.ROW_GROUP,
                                       64, shift=lin.unsigned_shift, lora_down=st["prep"][lname]["l2"],
                                       layout=self._lay4(M), codes=o["codes"], scales=o["scales"],
                                       lora_act=o["la"])

    def launch_gemm(self, si, lin, key, w_override=None):
        """w_override: (weights, w_layout) to run the GEMM kernel on weights
        already expanded to fp6 fragments (timing of the GEMM kernel alone)."""
        cr = self.cr
        st = self.sets[si]
        o, p, y = st["rq"][key], st["prep"][lin.name], st["out"][lin.name]
        M, N, K = lin.M, lin.N, lin.K
        wq, wlay = (p["w"], cr.LAYOUT.TILED) if w_override is None else w_override
        if lin.fmt == "w4a4":
            cr.w4a4_gemm(o["codes"], o["scales"], 0, wq, p["ws"], p.get("w_gran", 0), M, N, K, out=y, w_layout=wlay,
                         workspace=st["gws_c"][lin.chain])
        elif lin.fmt == "a8w4":
            cr.w4a4_gemm(o["codes"], o["scales"], cr.GRAN.ROW, p["w"], p["ws"], 0, M, N, K, out=y,
                         a_layout=cr.LAYOUT.INT8)
        elif lin.fmt == "int8":
            a8, s8 = (o["codes8"], o["scales8"]) if "codes8" in o else (o["codes"], o["scales"])
            cr.int8_tensorwise_gemm(a8, s8, p["w"], p["ws"], M, N, K, out=y)
        elif lin.fmt == "w4a8":
            cr.w4a8_gemm(o["codes"], o["scales"], cr.GRAN.ROW, p["w"], p["ws"], p["wz"], M, N, K, out=y)
        else:
            cr.w4a4_gemm(o["codes"], o["scales"], 2, wq, p["ws"], 2, M, N, K,
                         a_unsigned=lin.unsigned_shift != 0.0, a_shift=lin.unsigned_shift, w_sum=p["wsum"],
                         lora_act=o["la"], lora_up=p["l1"], out=y, w_layout=wlay, workspace=st["gws_c"][lin.chain])

    # ------------------------------------------------------------------
    def step_serial(self, i):
        """one step on one stream, every call in order (expansions inside the GEMM calls)"""
        for _, fn in self.order:
            fn(i % self.nsets)

    def step(self, i):
        """one step on the runner's schedule: "serial" (step_serial) or
        "chains": chain 0 on the launch stream, the others on side streams
        that start after an event recorded at the step's start and join the
        launch stream before the step ends (the next step starts after the
        whole of this one); between phases every chain waits for all the
        others; launches are issued round robin over the chains."""
        if self.schedule == "serial":
            self.step_serial(i)
            return
        torch = self.torch
        si = i % self.nsets
        main = self.stream
        streams = [main] + self.side
        start = torch.cuda.Event()
        start.record(main)
        for s in self.side:
            s.wait_event(start)
        for k, ph in enumerate(self.phases):
            if k > 0:                       # every chain waits for every chain's previous phase
                evs = []
                for s in streams:
                    ev = torch.cuda.Event()
                    ev.record(s)
                    evs.append(ev)
                for s in streams:
                    for t, ev in zip(streams, evs):
                        if t is not s:
                            s.wait_event(ev)
            lists = [self.corder[ph][c] for c in self.chains]
            for pos in range(max(len(l) for l in lists)):
                for s, l in zip(streams, lists):
                    if pos < len(l):
                        with torch.cuda.stream(s):
                            l[pos](si)
        for s in self.side:
            ev = torch.cuda.Event()
            ev.record(s)
            main.wait_event(ev)

    def _events(self, n):
        return [self.torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def time_steps(self, steps, warmup, schedule=None):
        """ms per step on `schedule` ("serial" or "chains"; None: the runner's)"""
        torch = self.torch
        keep = self.schedule
        if schedule is not None and len(self.chains) > 1:
            self.schedule = schedule
        step = self.step
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = self._events(2)
        e0.record(self.stream)
        for i in range(steps):
            step(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        self.schedule = keep
        return e0.elapsed_time(e1) / steps

    def shader_clock(self, fn, calls):
        """Shader clock (MHz) while `calls` launches of fn(i) keep the GPU busy:
        the current clock of every XCD from the GPU's metrics table (amdsmi),
        read from a host thread about every 2 ms from the fifth to the
        nine-tenths launch (untimed). None when amdsmi is not available."""
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:
            return None
        import threading
        torch = self.torch
        fn(0)
        torch.cuda.synchronize()
        first, last = calls // 5, (9 * calls) // 10
        e_start, e_stop = torch.cuda.Event(), torch.cuda.Event()
        stop_recorded = threading.Event()          # an event not yet recorded reads as complete
        samples = []

        def poll():
            while not e_start.query():
                time.sleep(0.0005)
            while not (stop_recorded.is_set() and e_stop.query()):
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    v = m.get("current_gfxclks")
                    if not isinstance(v, list):
                        v = [m.get("current_gfxclk")]
                    v = [x for x in v if isinstance(x, int) and 0 < x < 65535]
                    if v:
                        samples.append(v)
                except Exception:
                    pass
                time.sleep(0.002)

        th = threading.Thread(target=poll, daemon=True)
        for i in range(calls):
            fn(i)
            if i == first:
                e_start.record(self.stream)
                if not th.is_alive():
                    th.start()
            if i == last:
                e_stop.record(self.stream)
                stop_recorded.set()
        torch.cuda.synchronize()
        th.join()
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass
        if not samples:
            return None
        flat = [x for v in samples for x in v]
        return {"mean": round(sum(flat) / len(flat)), "min": min(flat), "max": max(flat),
                "readings": len(samples), "xcds": max(len(v) for v in samples)}

    def per_call(self, reps):
        """mean us of every call inside whole steps (events around each call)."""
        np, torch = self.np, self.torch
        per = {lab: [] for lab, _ in self.order}
        for r in range(reps):
            ev = self._events(len(self.order) + 1)
            ev[0].record(self.stream)
            for i, (_, fn) in enumerate(self.order):
                fn(r % self.nsets)
                ev[i + 1].record(self.stream)
            torch.cuda.synchronize()
            for i, (lab, _) in enumerate(self.order):
                per[lab].append(ev[i].elapsed_time(ev[i + 1]) * 1e3)
        return {lab: float(np.mean(v)) for lab, v in per.items()}

    def back_to_back(self, fn, reps, batches=1, warm=2):
        """us per launch of fn(set index) launched reps times back to back over
        the sets after `warm` untimed launches: the mean of one batch, or the
        median over `batches` such batches."""
        np, torch = self.np, self.torch
        for i in range(warm):
            fn(i % self.nsets)
        torch.cuda.synchronize()
        per = []
        for _ in range(batches):
            e0, e1 = self._events(2)
            e0.record(self.stream)
            for i in range(reps):
                fn(i % self.nsets)
            e1.record(self.stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / reps)
        return float(np.median(per))

    def gemm_kernel_fn(self, lin):
        """fn(set index) launching the GEMM kernel of layer `lin` alone. For a
        W4A4 layer on fp6 codes the weights are first expanded into each
        set's workspace by an ordinary call; the returned fn then runs the
        call on those fp6 fragments (no expansion pass)."""
        cr = self.cr
        key = [k for l, k in self.gemm_plan if l.name == lin.name][0]
        for si in range(self.nsets):
            self.launch_rq(si, key)
        if lin.fmt not in ("w4a4", "w4a4_g64") or not self.f6_codes(lin.M):
            return lambda si: self.launch_gemm(si, lin, key)
        exp = []
        for si in range(self.nsets):
            self.launch_gemm(si, lin, key)     # fills set si's workspace with the expanded weights
            n = (lin.N // 32) * (lin.K // 64) * 1536
            exp.append(self.sets[si]["gws_c"][lin.chain][:n].view(lin.N // 32, lin.K // 64, 1536))
        self.torch.cuda.synchronize()
        return lambda si: self.launch_gemm(si, lin, key, (exp[si], cr.LAYOUT.F6))

    def gemm_kernel_alone(self, lin, reps, batches=1, warm=2):
        """us of the GEMM kernel of layer `lin` alone, back to back (see back_to_back)."""
        return self.back_to_back(self.gemm_kernel_fn(lin), reps, batches, warm)

    def gemm_kernel_median(self, lin):
        """us of the GEMM kernel of layer `lin` alone: the median over 7 batches
        of at least 50 back-to-back launches (enough for ~10 ms each), after 10
        untimed launches."""
        fn = self.gemm_kernel_fn(lin)
        once = self.back_to_back(fn, 5)
        return self.back_to_back(fn, max(50, int(1e4 / once)), batches=7, warm=10)

    def ops(self):
        return sum(2.0 * l.M * l.N * l.K for l in self.w.linears)


def run(name, steps, warmup, cores="fp6", rot=256, extra=None):
    """One JSON line for workload `name` (bench.py --workload NAME); extra(line)
    may add fields (bench.py's CPU baseline) before it is printed."""
    if name == "merge":
        return run_merge(steps, warmup)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    r = Runner(name, cores, rot=rot)
    ms = r.time_steps(steps, warmup)
    ms_chains = r.time_steps(steps, warmup, schedule="chains") if len(r.chains) > 1 else None
    kern = r.per_call(max(3, steps // 2))
    layers = {}
    for lin, _ in r.gemm_plan:
        us = kern[f"gemm:{lin.name}"]
        d = {"us": round(us, 2), "TOPS": round(2.0 * lin.M * lin.N * lin.K / us / 1e6, 1),
             "GBps": round(gemm_bytes(lin) / us / 1e3, 1)}
        layers[lin.name] = d
    rqs = {}
    for key in r.rq_plan:
        x_id, kind, _ = key
        M, K = r.w.acts[x_id][0], r.w.acts[x_id][1]
        us = kern[f"rq:{x_id}:{kind}"]
        rqs[f"{x_id}:{kind}"] = {"us": round(us, 2), "GBps": round(rq_bytes(M, K, kind) / us / 1e3, 1)}
    dom = max(layers, key=lambda n: layers[n]["us"])
    dlin = [l for l in r.w.linears if l.name == dom][0]
    roof = gemm_roofline(dlin, r.gemm_kernel_median(dlin), cores)
    roof["kernel"] = (f"GEMM kernel of {dom} ({dlin.M}x{dlin.N}x{dlin.K}, {dlin.fmt}), alone, back to back "
                      f"(median of 7 batches)")
    eff = r.ops() / (ms * 1e-3) / 1e12
    line = {
        "metric": "effective TOPS of fused rotate+quant+W4 GEMM (% INT8 MFMA peak); GB/s",
        "value": round(eff, 2), "unit": "TOPS", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_chains_on_streams": None if ms_chains is None else round(ms_chains, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 / int8 codes (exact integer products)", "data": "synthetic",
        "config": {"workload": r.w.name, "layers": len(r.w.linears), "total_GOP": round(r.ops() / 1e9, 1),
                   "w4a4_matrix_cores": cores, "buffer_sets": r.nsets, "convrot_group": rot},
        "pct_int8_peak": round(100.0 * eff / INT8_PEAK_TOPS, 2),
        "gemm": layers, "rotate_quantize": rqs,
        "dominant_gemm": {"layer": dom, **layers[dom]},
        "roofline": roof,
        "setup_s": round(r.setup_s, 1),
    }
    del r
    if extra is not None:
        extra(line)
    print(json.dumps(line))


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
    moved = q_bytes + 2 * N * K + 2 * N * K + q_bytes + (N * K // 2 + N * K // 16 * 3) + R * (N + K) * 2
    print(json.dumps({
        "metric": "LoRA merge into a quantized weight (dequantize + rank-64 delta + requantize + pack)",
        "value": round(ms, 4), "unit": "ms per merge", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "higher_is_better": False, "data": "synthetic",
        "config": {"workload": "W4A8 asym g16 weight 12288x3072, ConvRot 256, LoRA rank 64"},
        "GBps": round(moved / ms / 1e6, 1)}))
