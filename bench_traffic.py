"""HBM traffic of the benchmark's dominant kernel (the GEMM kernel of one
layer of the mixed MMDiT block; default img_mlp_up on the fp6 matrix
cores), from rocprofv3 counters, calibrated against a plain copy kernel.

Subcommands:

  run [LAYER] [fp6|int8]
             the profiled workload: a copy kernel of known size (torch's
             elementwise negation of a 256 MiB bf16 tensor into another:
             256 MiB read, 256 MiB written), then the layer's GEMM kernel
             alone (weights already expanded into fp6 fragments), LAUNCHES
             times over the benchmark's two buffer sets. Run it once under
             `rocprofv3 --pmc FETCH_SIZE` and once under
             `rocprofv3 --pmc WRITE_SIZE` (one counter group per pass).

  summarize TF TW [LAYER] [fp6|int8]
             reads the two counter CSVs and writes profiles/<name>.json (read
             by bench.py for roofline.traffic) and a short .md summary.

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) count L2 <-> memory-fabric
traffic. Each is scaled by the same counter's reading for the copy kernel
divided by the copy's known bytes, so `hbm_bytes_per_launch` is in the units
the copy kernel calibrates. Only the last LAUNCHES dispatches of the GEMM
kernel are counted (the earlier ones belong to the weight expansion calls).

Commands (from /tmp with TMPDIR=/tmp; OUT = a directory for the counter output):
  rocprofv3 --pmc FETCH_SIZE -d $OUT/tf -o tf --output-format csv -- python3 $REPO/bench_traffic.py run
  rocprofv3 --pmc WRITE_SIZE -d $OUT/tw -o tw --output-format csv -- python3 $REPO/bench_traffic.py run
  python3 $REPO/bench_traffic.py summarize $OUT/tf $OUT/tw
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
KERNEL = {"fp6": "gemm_f6_kernel", "int8": "gemm_w4a4"}


def _args(argv):
    layer, cores = "img_mlp_up", "fp6"
    for a in argv:
        if a in ("fp6", "int8"):
            cores = a
        else:
            layer = a
    return layer, cores


def _out(cores, ext):
    return os.path.join(ROOT, "profiles", bench.TRAFFIC_PROFILE[cores].replace(".json", ext))


def run(layer, cores):
    import torch
    dev = torch.device("cuda:0")
    n = COPY_MIB * (1 << 20) // 2
    a = torch.randn(n, device=dev).to(torch.bfloat16)
    b = torch.empty_like(a)
    for _ in range(4):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b
    r = bw.Runner("c4", cores)
    lin = [l for l in r.w.linears if l.name == layer][0]
    fn = r.gemm_kernel_fn(lin)
    for i in range(LAUNCHES):
        fn(i % r.nsets)
    torch.cuda.synchronize()
    print(f"ran {LAUNCHES} launches of the {layer} GEMM kernel over {r.nsets} buffer sets", flush=True)


def _read(dirname, counter, cores):
    f = glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter CSV under {dirname}")
    copy, gemm = [], []
    for r in csv.DictReader(open(f[0])):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"]) * 1024.0          # KiB -> bytes
        name = r["Kernel_Name"]
        if "neg_kernel" in name or ("elementwise" in name and "neg" in name.lower()):
            copy.append(v)
        elif KERNEL[cores] in name:
            gemm.append((int(r.get("Dispatch_Id", len(gemm))), v))
    if not copy or not gemm:
        raise SystemExit(f"{counter}: copy or GEMM dispatches missing in {f[0]}")
    gemm = [v for _, v in sorted(gemm)][-LAUNCHES:]
    return copy, gemm


def summarize(dfetch, dwrite, layer, cores):
    import workloads as wl
    copy_bytes = COPY_MIB * (1 << 20)
    cf, gf = _read(dfetch, "FETCH_SIZE", cores)
    cw, gw = _read(dwrite, "WRITE_SIZE", cores)
    # the copy reads and writes its size once; the first dispatches may touch cold pages
    kf = sorted(cf)[len(cf) // 2] / copy_bytes
    kw = sorted(cw)[len(cw) // 2] / copy_bytes
    fetch = sum(gf) / len(gf) / kf
    write = sum(gw) / len(gw) / kw
    lin = [l for l in wl.CONFIGS["c4"]().linears if l.name == layer][0]
    alg = int(bw.gemm_bytes(lin))
    kname = ("gemm_f6_kernel (fp6 E2M3 operands, weights expanded from 4-bit tiles)" if cores == "fp6"
             else "int8-core W4A4 GEMM (4-bit operands widened to int8)")
    d = {
        "kernel": f"{kname}, layer {layer} ({lin.M}x{lin.N}x{lin.K}, tensorwise, bf16 out)",
        "layer": layer, "fmt": lin.fmt, "M": lin.M, "N": lin.N, "K": lin.K, "cores": cores,
        "source_sha": bench.source_sha(bench.GEMM_SOURCES[cores]),
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "hbm_bytes_per_launch": round(fetch) + round(write),
        "algorithmic_bytes_per_launch": alg,
        "copy_calibration": {"bytes": copy_bytes, "fetch_factor": round(kf, 4), "write_factor": round(kw, 4)},
        "launches_counted": len(gf),
    }
    arg = f" {layer} {cores}"
    with open(_out(cores, ".json"), "w") as f:
        json.dump(d, f, indent=1)
    with open(_out(cores, ".md"), "w") as f:
        f.write(f"# HBM traffic: GEMM kernel of {layer} ({lin.M}x{lin.N}x{lin.K}) on the {cores} matrix cores\n\n")
        f.write("Commands (from /tmp with TMPDIR=/tmp, REPO = repository root, OUT = the counter output directory):\n\n")
        f.write("    rocprofv3 --pmc FETCH_SIZE -d $OUT/tf -o tf --output-format csv -- "
                f"python3 $REPO/bench_traffic.py run{arg}\n")
        f.write("    rocprofv3 --pmc WRITE_SIZE -d $OUT/tw -o tw --output-format csv -- "
                f"python3 $REPO/bench_traffic.py run{arg}\n")
        f.write(f"    python3 $REPO/bench_traffic.py summarize $OUT/tf $OUT/tw{arg}\n\n")
        f.write(f"Copy-kernel calibration ({COPY_MIB} MiB read + {COPY_MIB} MiB written by torch.neg): "
                f"FETCH_SIZE reads {kf:.4f} x the bytes read, WRITE_SIZE {kw:.4f} x the bytes written.\n\n")
        f.write("| per GEMM launch | bytes |\n|---|---|\n")
        f.write(f"| fetched (calibrated) | {fetch/1e6:.2f} MB |\n")
        f.write(f"| written (calibrated) | {write/1e6:.2f} MB |\n")
        f.write(f"| total | {(fetch + write)/1e6:.2f} MB |\n")
        f.write(f"| algorithmic (4-bit activation codes + 4-bit weights + bf16 output) | {alg/1e6:.2f} MB |\n\n")
        f.write(f"Kernel source hash: `{d['source_sha']}` ({len(gf)} launches counted).\n")
    print(json.dumps(d))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run(*_args(sys.argv[2:]))
    elif len(sys.argv) >= 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3], *_args(sys.argv[4:]))
    else:
        print(__doc__)
        sys.exit(2)
