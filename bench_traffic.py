"""HBM traffic of the benchmark's dominant kernel (the M=4096 W4A4 GEMM,
on the fp6 matrix cores by default, or the int8-core kernel with a trailing
`int8` argument), from rocprofv3 counters, calibrated against a plain copy
kernel.

Two subcommands:

  run        the profiled workload: a copy kernel of known size
             (torch's elementwise negation of a 256 MiB bf16 tensor into
             another: 256 MiB read, 256 MiB written), then the GEMM of
             bench.py over its rotating buffer sets. Run it once under
             `rocprofv3 --pmc FETCH_SIZE` and once under
             `rocprofv3 --pmc WRITE_SIZE` (one counter group per pass).

  summarize  reads the two counter CSVs and writes
             profiles/w4a4_f6_gemm_m4096_n3072_k3072_traffic.json (int8:
             profiles/w4a4_gemm_m4096_n3072_k3072_traffic.json; read by
             bench.py for roofline.traffic) and a short .md summary.

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) count L2 <-> memory-fabric
traffic. Each is scaled by the same counter's reading for the copy kernel
divided by the copy's known bytes, so `hbm_bytes_per_launch` is in the
units the copy kernel calibrates.

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

COPY_MIB = 256
LAUNCHES = 10
KERNEL = {"fp6": "gemm_f6_kernel", "int8": "gemm_w4a4"}


def _out(ext):
    return os.path.join(ROOT, "profiles", bench.TRAFFIC_PROFILE[bench.CORES].replace(".json", ext))


def run():
    import torch
    import w4a8_rotated_quantized_amd as cr
    dev = torch.device("cuda:0")
    n = COPY_MIB * (1 << 20) // 2
    a = torch.randn(n, device=dev).to(torch.bfloat16)
    b = torch.empty_like(a)
    for _ in range(4):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    sets = bench.setup(dev)
    for i in range(len(sets)):
        bench.rq_big(cr, sets[i])
    torch.cuda.synchronize()
    for i in range(LAUNCHES):
        bench.gemm_big(cr, sets[i % len(sets)])
    torch.cuda.synchronize()
    print(f"ran {LAUNCHES} GEMM launches over {len(sets)} buffer sets", flush=True)


def _read(dirname, counter):
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
        elif KERNEL[bench.CORES] in name:
            gemm.append(v)
    if not copy or not gemm:
        raise SystemExit(f"{counter}: copy or GEMM dispatches missing in {f[0]}")
    return copy, gemm


def summarize(dfetch, dwrite):
    copy_bytes = COPY_MIB * (1 << 20)
    cf, gf = _read(dfetch, "FETCH_SIZE")
    cw, gw = _read(dwrite, "WRITE_SIZE")
    # the copy reads and writes its size once; the first dispatches may touch cold pages
    kf = sorted(cf)[len(cf) // 2] / copy_bytes
    kw = sorted(cw)[len(cw) // 2] / copy_bytes
    fetch = sum(gf) / len(gf) / kf
    write = sum(gw) / len(gw) / kw
    code_bytes = (3 * bench.K // 4) if bench.CORES == "fp6" else bench.K // 2   # per row: fp6 or int4 codes
    alg = bench.M_BIG * code_bytes + bench.N * code_bytes + bench.M_BIG * bench.N * 2
    kname = ("gemm_f6_kernel<256, 192, ...> (fp6 E2M3 operands)" if bench.CORES == "fp6"
             else "gemm_w4a4_lds_kernel (int4 operands widened to int8)")
    d = {
        "kernel": f"{kname} (M=4096, N=3072, K=3072, tensorwise, bf16 out)",
        "source_sha": bench.source_sha(bench.GEMM_SOURCES[bench.CORES]),
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "hbm_bytes_per_launch": round(fetch + write),
        "algorithmic_bytes_per_launch": alg,
        "copy_calibration": {"bytes": copy_bytes, "fetch_factor": round(kf, 4), "write_factor": round(kw, 4)},
        "launches_counted": len(gf),
    }
    arg = "" if bench.CORES == "fp6" else " int8"
    with open(_out(".json"), "w") as f:
        json.dump(d, f, indent=1)
    with open(_out(".md"), "w") as f:
        f.write(f"# HBM traffic: W4A4 GEMM on the {bench.CORES} matrix cores, M=4096, N=K=3072 (benchmarked kernel)\n\n")
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
        f.write(f"| algorithmic (activation codes + packed weights + bf16 output) | {alg/1e6:.2f} MB |\n\n")
        f.write("Each of the 8 XCDs has its own 4 MB L2; with the XCD-aware tile map every XCD fetches the "
                "activation rows and weight columns of its part of the output, so operand bytes repeat across "
                "XCDs (served by the 256 MB last-level cache). The written bytes are the bf16 output.\n\n")
        f.write(f"Kernel source hash: `{d['source_sha']}` ({len(gf)} launches counted).\n")
    print(json.dumps(d))


if __name__ == "__main__":
    if sys.argv[-1] in ("fp6", "int8"):
        bench.CORES = sys.argv.pop()
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) == 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    else:
        print(__doc__)
        sys.exit(2)
