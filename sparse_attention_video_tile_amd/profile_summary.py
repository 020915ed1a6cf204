"""Summaries of rocprofv3 output for the profiles/ records.

    python -m sparse_attention_video_tile_amd.profile_summary RUN_DIR OUT_DIR

RUN_DIR holds what one profiling session of bench.py wrote:
  bench.json                 bench.py's JSON line, run without a profiler
  trace/bench_kernel_stats.csv
      rocprofv3 --kernel-trace --stats -d RUN_DIR/trace -o bench -f csv -- python3 bench.py
  FETCH_SIZE/run_counter_collection.csv, WRITE_SIZE/run_counter_collection.csv
      rocprofv3 --pmc <counter> --kernel-trace -d RUN_DIR/<counter> -o run -f csv --
          python3 bench.py --steps 2 --warmup 1 --cpu-budget 0 --dense-reps 1
          --compare-reps 1 --copy-reference

Writes, for the workload named in bench.json, a kernel-time table, an HBM
traffic table, and per path (fused, three_call) a JSON record of the bytes
per attention launch that bench.py reports as roofline.traffic while the
kernel sources are unchanged. Counter values are per dispatch, summed over
the XCD instances rocprofv3 lists; FETCH_SIZE and WRITE_SIZE are scaled by
what they read for the plain device copy (--copy-reference) of a q-sized
tensor, whose true size is known.
"""

from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = (
    "sparse_attention_video_tile_amd/csrc/sta_attention.hip",
    "sparse_attention_video_tile_amd/csrc/sta_geometry.h",
    "sparse_attention_video_tile_amd/csrc/sta_kernels.h",
)
TRACE_CMD = "rocprofv3 --kernel-trace --stats -d <outdir> -o bench -f csv -- python3 bench.py"
PMC_ARGS = "--steps 2 --warmup 1 --cpu-budget 0 --dense-reps 1 --compare-reps 1 --copy-reference"


def pmc_cmd(counter: str) -> str:
    return f"rocprofv3 --pmc {counter} --kernel-trace -d <outdir> -o run -f csv -- python3 bench.py {PMC_ARGS}"


def source_sha256(root: str = ROOT) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(root, f), "rb").read())
    return h.hexdigest()


def short_name(n: str) -> str:
    n = n.replace("sta::(anonymous namespace)::", "").replace("void ", "")
    n = n.replace("(AttnParams)", "").replace("(ReorderParams)", "")
    if "distribution_elementwise" in n:
        return "torch randn (input generation)"
    if "bfloat16_copy_kernel" in n:
        return "torch float32->bf16 cast (input generation)"
    if "copyBuffer" in n:
        return "HIP runtime copyBuffer (plain device copy)"
    return n[:90]


def role(name: str) -> str:
    if "attn_bf16_kernel" in name or "attn_f32_kernel" in name:
        args = name[name.index("<") + 1:name.index(">")].split(",")
        dense, raster = args[-2].strip() == "true", args[-1].strip() == "true"
        if dense:
            return "dense comparator"
        return "STA forward, raster order (fused path)" if raster else "STA forward, tile-major (three-call path)"
    if "reorder_kernel" in name:
        return "tile reorder / restore (one tensor)"
    return ""


def per_dispatch(path: str):
    agg = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        agg[k] = agg.get(k, 0.0) + float(r["Counter_Value"])
    return agg


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) != 2:
        print(__doc__, file=sys.stderr)
        return 2
    run, out = argv
    bench = json.load(open(os.path.join(run, "bench.json")))
    cfg = bench["config"]
    wl = cfg["workload"]
    B, heads, d = cfg["B"], cfg["heads"], cfg["head_dim"]
    S = cfg["volume"][0] * cfg["volume"][1] * cfg["volume"][2]
    elem = 2 if bench["dtype"] == "bf16" else 4
    tensor = B * heads * S * d * elem
    title = f"{wl} ({bench['dtype']}, B={B}, {heads} heads, d={d})"

    # Kernel time.
    rows = list(csv.DictReader(open(os.path.join(run, "trace", "bench_kernel_stats.csv"))))
    L = [f"# Kernel time, bench.py on {title}\n", "Command (repo root, MI355X, ROCm 7.2):\n",
         f"```\n{TRACE_CMD}\n```\n",
         "bench.py defaults: 3 warm-up + 20 timed steps of the fused path (one raster-order STA launch), "
         "then 1 + 3 steps of the three-call path (reorder q, k, v; tile-major STA; restore), then "
         "1 + 2 dense-comparator launches at the same shape.\n",
         "| kernel | role | calls | average (ms) | min (ms) | max (ms) | share |",
         "|---|---|---|---|---|---|---|"]
    for r in rows:
        L.append(f"| `{short_name(r['Name'])}` | {role(r['Name'])} | {r['Calls']} | "
                 f"{float(r['AverageNs']) / 1e6:.3f} | {float(r['MinNs']) / 1e6:.3f} | "
                 f"{float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.1f}% |")
    rf = bench["roofline"]
    L += ["", f"bench.py's HIP-event average for the timed kernel ({rf['kernel']}) in the same command "
          f"without the profiler: {rf['launch_ms']:.3f} ms, {rf['achieved']:.1f} TFLOP/s of algorithmic "
          f"work ({cfg['algorithmic_tflop_per_step']:.4f} TFLOP per launch), "
          f"{100 * rf['frac']:.1f}% of the {rf['peak']:.0f} TFLOP/s dense peak."]
    name = f"attn_{bench['dtype']}_{wl}_kernel_stats.md"
    open(os.path.join(out, name), "w").write("\n".join(L) + "\n")

    # Traffic.
    fetch = per_dispatch(os.path.join(run, "FETCH_SIZE", "run_counter_collection.csv"))
    write = per_dispatch(os.path.join(run, "WRITE_SIZE", "run_counter_collection.csv"))
    cf = [v for (_, n), v in fetch.items() if "copyBuffer" in n][0]
    cw = [v for (_, n), v in write.items() if "copyBuffer" in n][0]
    fscale, wscale = tensor / 1024 / cf, tensor / 1024 / cw

    def summarize(pred):
        fs = [v for (_, n), v in fetch.items() if pred(n)]
        ws = [v for (_, n), v in write.items() if pred(n)]
        return (sum(fs) / len(fs), sum(ws) / len(ws), len(fs)) if fs else None

    kernels = []
    for n in dict.fromkeys(n for (_, n) in fetch):
        if role(n):
            kernels.append(n)
    L = [f"# HBM-side traffic per launch, bench.py on {title}\n",
         "Commands (repo root), one counter per run:\n",
         f"```\n{pmc_cmd('FETCH_SIZE')}\n{pmc_cmd('WRITE_SIZE')}\n```\n",
         f"Calibration: `--copy-reference` runs one plain device copy of a q-sized tensor ({tensor} bytes "
         f"read and written). It reads FETCH_SIZE = {cf:.0f} KiB and WRITE_SIZE = {cw:.0f} KiB, so "
         f"bytes = FETCH_SIZE x {fscale:.3f} KiB and WRITE_SIZE x {wscale:.3f} KiB.\n",
         "| kernel | role | launches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read GB (scaled) | "
         "written GB (scaled) | algorithmic GB (read + written) |",
         "|---|---|---|---|---|---|---|---|"]
    records = {}
    for n in kernels:
        f, w, c = summarize(lambda x, n=n: x == n)
        alg = (tensor, tensor) if "reorder" in n else (3 * tensor, tensor)
        L.append(f"| `{short_name(n)}` | {role(n)} | {c} | {f:.0f} | {w:.0f} | "
                 f"{f * fscale * 1024 / 1e9:.3f} | {w * wscale * 1024 / 1e9:.3f} | "
                 f"{alg[0] / 1e9:.3f} + {alg[1] / 1e9:.3f} |")
        r = role(n)
        path = "fused" if "fused" in r else "three_call" if "three-call" in r else None
        if path:
            records[path] = {
                "kernel": short_name(n),
                "workload": wl,
                "path": path,
                "source_sha256": source_sha256(),
                "read_bytes_per_launch": f * fscale * 1024,
                "write_bytes_per_launch": w * wscale * 1024,
                "bytes_per_launch": f * fscale * 1024 + w * wscale * 1024,
                "algorithmic_bytes_per_launch": 4 * tensor,
                "fetch_kib_to_bytes": fscale * 1024,
                "write_kib_to_bytes": wscale * 1024,
                "commands": [pmc_cmd("FETCH_SIZE"), pmc_cmd("WRITE_SIZE")],
            }
    L += ["", "\"Algorithmic\" counts every input element once and every output element once "
          "(q, k, v read; o written). The attention kernels re-read K and V for every query tile "
          "whose window holds them; what the counters show is the traffic below L2 (HBM and the "
          "memory-side cache)."]
    open(os.path.join(out, f"attn_{bench['dtype']}_{wl}_traffic.md"), "w").write("\n".join(L) + "\n")
    for path, rec in records.items():
        fn = os.path.join(out, f"attn_{bench['dtype']}_{path}_{wl}_traffic.json")
        json.dump(rec, open(fn, "w"), indent=1)
    print(json.dumps({p: r["bytes_per_launch"] for p, r in records.items()}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
