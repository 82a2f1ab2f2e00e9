"""rocprofv3 counter summaries for the benchmark: HBM traffic, VALU and
matrix-core activity of every kernel of one mixed-MMDiT-block step, and the
HBM traffic of the dominant kernel that bench.py reports as roofline.traffic.

Subcommands:

  run [LAYER] [fp6|int8]
        the profiled program: the benchmark's block (bench_workloads.Runner,
        weights prepared first), then four launches of a plain copy kernel
        of known size (torch's elementwise negation of a 256 MiB bf16 tensor
        into another: 256 MiB read, 256 MiB written), one whole step, one
        more negation (marks the step's end), and finally the GEMM kernel of
        LAYER (default img_mlp_up) alone, LAUNCHES times, on weights already
        expanded into fp6 fragments. Run it once per counter group under
        `rocprofv3 --pmc ...` (one group per pass; see the commands below).

  summarize DIR... [LAYER] [fp6|int8]
        merges the counter CSVs of the passes by dispatch and writes
          profiles/c4_step_counters.md   every kernel of the step
          profiles/<traffic>.json / .md  the dominant kernel's HBM bytes
                                         (read by bench.py)

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) count L2 <-> memory-fabric
traffic; each is scaled by the same counter's reading for the copy kernel
divided by the copy's known bytes. Matrix-core utilisation is
SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs) (the per-dispatch
GRBM_GUI_ACTIVE sums the copies of the 8 XCDs); matrix ops are
SQ_INSTS_VALU_MFMA_MOPS_* x 512.

Commands (from /tmp with TMPDIR=/tmp; OUT = a directory for the counter output):
  rocprofv3 --pmc FETCH_SIZE -d $OUT/p1 -o p1 --output-format csv -- python3 $REPO/bench_traffic.py run
  rocprofv3 --pmc WRITE_SIZE -d $OUT/p2 -o p2 --output-format csv -- python3 $REPO/bench_traffic.py run
  rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_INSTS_LDS SQ_WAVES \\
            SQ_BUSY_CYCLES SQ_WAVE_CYCLES -d $OUT/p3 -o p3 --output-format csv -- python3 $REPO/bench_traffic.py run
  rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F6F4 \\
            SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_MFMA GRBM_GUI_ACTIVE \\
            -d $OUT/p4 -o p4 --output-format csv -- python3 $REPO/bench_traffic.py run
  python3 $REPO/bench_traffic.py summarize $OUT/p1 $OUT/p2 $OUT/p3 $OUT/p4
"""
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bench_workloads as bw  # noqa: E402

COPY_MIB = 256
LAUNCHES = 10
SIMDS = 1024
XCDS = 8                      # GRBM_GUI_ACTIVE per dispatch is the sum over the 8 XCDs' copies
KERNEL = {"fp6": "gemm_f6_kernel", "int8": "gemm_w4a4"}
COMMANDS = __doc__[__doc__.index("Commands"):].strip()


def _args(argv):
    layer, cores, rest = "img_mlp_up", "fp6", []
    for a in argv:
        if a in ("fp6", "int8"):
            cores = a
        elif os.path.isdir(a):
            rest.append(a)
        else:
            layer = a
    return layer, cores, rest


def _out(cores, ext):
    return os.path.join(ROOT, "profiles", bench.TRAFFIC_PROFILE[cores].replace(".json", ext))


def run(layer, cores):
    import torch
    dev = torch.device("cuda:0")
    r = bw.Runner("c4", cores, fuse=True)      # the step as bench.py runs it (fused Q/K calls)
    lin = [l for l in r.w.linears if l.name == layer][0]
    n = COPY_MIB * (1 << 20) // 2
    a = torch.randn(n, device=dev).to(torch.bfloat16)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(4):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    r.step(0)
    torch.cuda.synchronize()
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    fn = r.gemm_kernel_fn(lin)
    for i in range(LAUNCHES):
        fn(i % r.nsets)
    torch.cuda.synchronize()
    print(f"ran one step and {LAUNCHES} launches of the {layer} GEMM kernel", flush=True)


def _is_copy(name):
    return "neg_kernel" in name or ("elementwise" in name and "neg" in name.lower())


def _load(dirs):
    """dispatch id -> {"name", "grid", counter: value} merged over the passes
    (every pass runs the same program, so dispatch ids line up)."""
    disp = {}
    for d in dirs:
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter CSV under {d}")
        for row in csv.DictReader(open(f[0])):
            i = int(row["Dispatch_Id"])
            e = disp.setdefault(i, {"name": row["Kernel_Name"], "grid": int(row.get("Grid_Size", 0) or 0)})
            e[row["Counter_Name"]] = e.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return [disp[i] for i in sorted(disp)]


def _short(name):
    name = name.replace("void ", "").replace("(cr::GemmParams)", "").replace("(cr::RQParams)", "")
    return name.split("(")[0].replace("cr::", "")


def summarize(dirs, layer, cores):
    import workloads as wl
    rows = _load(dirs)
    copies = [i for i, e in enumerate(rows) if _is_copy(e["name"])]
    if len(copies) < 5:
        raise SystemExit("copy-kernel markers missing")
    copy_bytes = COPY_MIB * (1 << 20)
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = sorted(rows[i][c] * 1024.0 for i in copies[:4] if c in rows[i])
        cal[c] = v[len(v) // 2] / copy_bytes if v else None
    step = rows[copies[3] + 1:copies[4]]
    gemm = [e for e in rows[copies[4] + 1:] if KERNEL[cores] in e["name"]][-LAUNCHES:]

    def hbm(e, c):
        return e[c] * 1024.0 / cal[c] if (c in e and cal[c]) else None

    # ---- the dominant kernel's traffic (bench.py roofline.traffic) ----
    lin = [l for l in wl.CONFIGS["c4"]().linears if l.name == layer][0]
    alg = int(bw.gemm_bytes(lin))
    fetch = sum(hbm(e, "FETCH_SIZE") for e in gemm) / len(gemm)
    write = sum(hbm(e, "WRITE_SIZE") for e in gemm) / len(gemm)
    mops = [e.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0) + e.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0.0) for e in gemm]
    busy = [e["SQ_VALU_MFMA_BUSY_CYCLES"] / (e["GRBM_GUI_ACTIVE"] / XCDS * SIMDS) for e in gemm
            if e.get("GRBM_GUI_ACTIVE")]
    d = {
        "kernel": f"{KERNEL[cores]}, layer {layer} ({lin.M}x{lin.N}x{lin.K}, tensorwise, bf16 out)",
        "layer": layer, "fmt": lin.fmt, "M": lin.M, "N": lin.N, "K": lin.K, "cores": cores,
        "source_sha": bench.source_sha(bench.GEMM_SOURCES[cores]),
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "hbm_bytes_per_launch": round(fetch) + round(write),
        "algorithmic_bytes_per_launch": alg,
        "matrix_ops_per_launch": round(sum(mops) / len(mops) * 512) if mops else None,
        "mfma_busy_frac": round(sum(busy) / len(busy), 4) if busy else None,
        "copy_calibration": {"bytes": copy_bytes, "fetch_factor": round(cal["FETCH_SIZE"], 4),
                             "write_factor": round(cal["WRITE_SIZE"], 4)},
        "launches_counted": len(gemm),
    }
    arg = "" if (layer, cores) == ("img_mlp_up", "fp6") else f" {layer} {cores}"
    with open(_out(cores, ".json"), "w") as f:
        json.dump(d, f, indent=1)
    with open(_out(cores, ".md"), "w") as f:
        f.write(f"# HBM traffic and matrix-core activity: GEMM kernel of {layer} "
                f"({lin.M}x{lin.N}x{lin.K}), {cores} matrix cores\n\n")
        f.write("```\n" + COMMANDS.replace("bench_traffic.py run", "bench_traffic.py run" + arg)
                .replace("$OUT/p4\n", f"$OUT/p4{arg}\n") + "\n```\n\n")
        f.write(f"Copy-kernel calibration ({COPY_MIB} MiB read + {COPY_MIB} MiB written by torch.neg): "
                f"FETCH_SIZE reads {cal['FETCH_SIZE']:.4f} x the bytes read, WRITE_SIZE {cal['WRITE_SIZE']:.4f} x "
                f"the bytes written.\n\n")
        f.write("| per GEMM launch | value |\n|---|---|\n")
        f.write(f"| fetched (calibrated) | {fetch/1e6:.2f} MB |\n")
        f.write(f"| written (calibrated) | {write/1e6:.2f} MB |\n")
        f.write(f"| algorithmic (4-bit codes + 4-bit weights + bf16 output) | {alg/1e6:.2f} MB |\n")
        if d["matrix_ops_per_launch"]:
            f.write(f"| matrix ops (MOPS counter x 512) | {d['matrix_ops_per_launch']/1e9:.1f} G "
                    f"(2MNK = {2.0*lin.M*lin.N*lin.K/1e9:.1f} G) |\n")
        if d["mfma_busy_frac"] is not None:
            f.write(f"| matrix-core busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024)) | "
                    f"{100*d['mfma_busy_frac']:.1f} % |\n")
        f.write(f"\nKernel source hash: `{d['source_sha']}` ({len(gemm)} launches counted).\n")

    # ---- every kernel of one step ----
    with open(os.path.join(ROOT, "profiles", "c4_step_counters.md"), "w") as f:
        f.write("# Counters of every kernel of one mixed-MMDiT-block step (bench.py's default workload)\n\n")
        f.write("```\n" + COMMANDS + "\n```\n\n")
        f.write("HBM MB = FETCH_SIZE / WRITE_SIZE scaled by a copy kernel of known size (L2 misses: bytes from the "
                "last-level cache count too); VALU and MFMA instruction counts are per dispatch (wave "
                "instructions, all waves); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 "
                "SIMDs).\n\n")
        f.write("| # | kernel | grid | fetch MB | write MB | VALU insts (M) | MFMA insts (K) | matrix Gops | "
                "MFMA busy % |\n|---|---|---|---|---|---|---|---|---|\n")
        for k, e in enumerate(step):
            fm = hbm(e, "FETCH_SIZE")
            wm = hbm(e, "WRITE_SIZE")
            mo = sum(e.get(c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_INSTS_VALU_MFMA_MOPS_I8",
                                             "SQ_INSTS_VALU_MFMA_MOPS_F16")) * 512
            bz = (100 * e["SQ_VALU_MFMA_BUSY_CYCLES"] / (e["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
                  if e.get("GRBM_GUI_ACTIVE") else None)
            f.write(f"| {k} | `{_short(e['name'])}` | {e['grid']} | "
                    f"{'' if fm is None else f'{fm/1e6:.1f}'} | {'' if wm is None else f'{wm/1e6:.1f}'} | "
                    f"{e.get('SQ_INSTS_VALU', 0)/1e6:.2f} | {e.get('SQ_INSTS_MFMA', 0)/1e3:.1f} | {mo/1e9:.1f} | "
                    f"{'' if bz is None else f'{bz:.1f}'} |\n")
    print(json.dumps(d))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        layer, cores, _ = _args(sys.argv[2:])
        run(layer, cores)
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize":
        layer, cores, dirs = _args(sys.argv[2:])
        summarize(dirs, layer, cores)
    else:
        print(__doc__)
        sys.exit(2)
