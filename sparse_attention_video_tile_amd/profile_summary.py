"""Summaries of rocprofv3 output for the profiles/ records.

    python -m sparse_attention_video_tile_amd.profile_summary RUN_DIR OUT_DIR

RUN_DIR holds what one profiling session of bench.py wrote:
  bench.json                 bench.py's JSON line, run without a profiler
  trace/bench_kernel_stats.csv
      rocprofv3 --kernel-trace --stats -d RUN_DIR/trace -o bench -f csv -- python3 bench.py --cpu none
  FETCH_SIZE/run_counter_collection.csv, WRITE_SIZE/run_counter_collection.csv
      rocprofv3 --pmc <counter> --kernel-trace -d RUN_DIR/<counter> -o run -f csv --
          python3 bench.py --steps 2 --warmup 1 --cpu none --dense-reps 1
          --compare-reps 1 --copy-reference
  MFMA/run_counter_collection.csv (optional)
      rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --kernel-trace
          -d RUN_DIR/MFMA -o run -f csv -- python3 bench.py <same arguments>
  PIPE/run_counter_collection.csv, LDS/run_counter_collection.csv (optional)
      the same with the PIPE_COUNTERS and LDS_COUNTERS sets below (one pass each)

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
    "sparse_attention_video_tile_amd/csrc/sta_attn_common.h",
    "sparse_attention_video_tile_amd/csrc/sta_geometry.h",
    "sparse_attention_video_tile_amd/csrc/sta_kernels.h",
    "sparse_attention_video_tile_amd/csrc/sta_plan.h",
)
TRACE_CMD = "rocprofv3 --kernel-trace --stats -d <outdir> -o bench -f csv -- python3 bench.py --cpu none"
PMC_ARGS = "--steps 2 --warmup 1 --cpu none --dense-reps 1 --compare-reps 1 --copy-reference"


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE"
# Issue and wait profile; LDS profile (each within one pass's counter limits).
PIPE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU "
                 "SQ_INSTS_MFMA SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_WAVE_CYCLES GRBM_GUI_ACTIVE")
LDS_COUNTERS = ("SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS "
                "SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")
N_CU = 256          # MI355X compute units
SIMD_PER_CU = 4


def pmc_cmd(counter: str) -> str:
    return f"rocprofv3 --pmc {counter} --kernel-trace -d <outdir> -o run -f csv -- python3 bench.py {PMC_ARGS}"


def strip_comments(text: str) -> str:
    """C/C++ source without its comments and blank lines, trailing spaces cut:
    what the compiler sees, so that an edit of a comment leaves it unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln) + "\n"


def source_sha256(root: str = ROOT, read=None) -> str:
    """Hash of the kernel sources' code (comments removed). A counter record
    whose hash differs was taken from other kernels."""
    read = read or (lambda f: open(os.path.join(root, f), encoding="utf-8").read())
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(strip_comments(read(f)).encode())
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
    if "delta_kernel" in n and n.startswith("_Z"):   # reported mangled
        return "delta_kernel"
    return n[:90]


def role(name: str) -> str:
    """What a kernel is, from its name and template arguments."""
    if "bwd_dkdv_pair_kernel" in name:
        return "STA backward, key side (dK, dV), paired waves"
    if "bwd_dkdv_kernel" in name or "bwd_f32_dkdv" in name:
        return "STA backward, key side (dK, dV)"
    if "bwd_dq_kernel" in name or "bwd_f32_dq" in name:
        return "STA backward, query side (dQ)"
    if "delta_kernel" in name:
        return "STA backward, D = rowsum(dO * O)"
    if "attn_bf16_kernel" in name:
        a = _targs(name)
        # <D, WAVES, RB, BN, DENSE, RASTER, LSE_ONLY, PAD, PLANE, FULL, QK8, RECALL>
        dense, raster = a[4] == "true", a[5] == "true"
        lse_only = len(a) > 6 and a[6] == "true"
        pad = len(a) > 7 and a[7] == "true"
        qk8 = len(a) > 10 and a[10] == "true"
        small = a[1] == "4" and a[2] == "1"   # 4 waves of 16 rows: 64-row items
        ksplit = a[1] == "8" and a[2] == "1"  # two groups of 4 waves on 64 rows (a split last round)
        what = "dense comparator" if dense else (
            "STA forward, raster order (fused path)" if raster else "STA forward, tile-major (three-call path)")
        if lse_only:
            what += ", log-sum-exp only (recall)"
        if pad:
            what += ", padded grid"
        if qk8:
            what += ", fp8 q and k"
        if len(a) > 11 and a[11] == "true":
            what += ", one pass over all candidate windows"
        if small:
            what += ", 64-row items"
        if ksplit:
            what += ", 64-row items, keys split over two wave groups"
        return what
    if "attn_f32_kernel" in name:
        return "STA forward, float32"
    if "reorder_kernel" in name:
        return "tile reorder / restore (one tensor)"
    if "recall_reduce" in name:
        return "window recall reduction"
    return ""


def _targs(name: str):
    return [x.strip() for x in name[name.index("<") + 1:name.index(">")].split(",")]


def is_headline(name: str) -> bool:
    """The fused (raster-order) forward kernel that bench.py times, whole-tile
    items: not the log-sum-exp-only, padded or 64-row variants."""
    return role(name) == "STA forward, raster order (fused path)"


def is_headline_tail(name: str) -> bool:
    """The second launch of a headline step: the last round's items as 64-row
    items (absent when the work items fill every round)."""
    return role(name).startswith("STA forward, raster order (fused path), 64-row items")


def step_dispatches(ids_names):
    """[(main dispatch id, tail dispatch id or None)] of the headline steps,
    in order, from (dispatch id, kernel name) pairs: a tail launch belongs to
    the main launch it directly follows."""
    steps = []
    for d, n in sorted(ids_names):
        if is_headline(n):
            steps.append([d, None])
        elif is_headline_tail(n) and steps and steps[-1][1] is None and d == steps[-1][0] + 1:
            steps[-1][1] = d
    return [tuple(x) for x in steps]


N_XCD = 8   # rocprofv3 reports GRBM_GUI_ACTIVE summed over the XCDs


def per_dispatch(path: str, counter: str = None):
    agg = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        if counter is not None and r.get("Counter_Name") != counter:
            continue
        k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        agg[k] = agg.get(k, 0.0) + float(r["Counter_Value"])
    return agg


def all_counters(path: str):
    """{(dispatch, kernel): {counter: value summed over instances}}."""
    agg = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        c = agg.setdefault(k, collections.defaultdict(float))
        c[r["Counter_Name"]] += float(r["Counter_Value"])
    return agg


def pipeline_summary(run: str, out: str, bench: dict, title: str) -> None:
    """Per kernel: where the SIMDs' cycles go (MFMA, VALU, both, waiting) and
    how hard the LDS is driven, from the PIPE and LDS counter passes."""
    ppath = os.path.join(run, "PIPE", "run_counter_collection.csv")
    lpath = os.path.join(run, "LDS", "run_counter_collection.csv")
    if not (os.path.exists(ppath) and os.path.exists(lpath)):
        return
    pipe, lds = all_counters(ppath), all_counters(lpath)

    def mean_by_kernel(agg, fn):
        vals = collections.defaultdict(list)
        for (_, n), c in agg.items():
            if role(n) and c.get("GRBM_GUI_ACTIVE"):
                vals[n].append(fn(c))
        return {n: sum(v) / len(v) for n, v in vals.items()}

    simd_cycles = lambda c: c["GRBM_GUI_ACTIVE"] / N_XCD * N_CU * SIMD_PER_CU
    cu_cycles = lambda c: c["GRBM_GUI_ACTIVE"] / N_XCD * N_CU
    cols = {
        "mfma": mean_by_kernel(pipe, lambda c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles(c)),
        "valu": mean_by_kernel(pipe, lambda c: 4 * c["SQ_ACTIVE_INST_VALU"] / simd_cycles(c)),
        "coexec": mean_by_kernel(pipe, lambda c: c["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cycles(c)),
        "wait": mean_by_kernel(pipe, lambda c: c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]),
        "waitinst": mean_by_kernel(pipe, lambda c: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
        "vpm": mean_by_kernel(pipe, lambda c: c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"]
                              if c["SQ_INSTS_MFMA"] else float("nan")),
        "ldsbw": mean_by_kernel(lds, lambda c: 64 * c["SQ_INSTS_LDS_LOAD_BANDWIDTH"] / cu_cycles(c)),
        "conf": mean_by_kernel(lds, lambda c: c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1)),
        "ldswait": mean_by_kernel(lds, lambda c: c["SQ_WAIT_INST_LDS"] / max(c["SQ_ACTIVE_INST_LDS"], 1)),
    }
    L = [f"# Issue, wait and LDS profile per kernel, bench.py on {title}\n",
         "Commands (repo root), one pass each:\n",
         f"```\nrocprofv3 --pmc {PIPE_COUNTERS} --kernel-trace -d <outdir> -o run -f csv -- "
         f"python3 bench.py {PMC_ARGS}\n"
         f"rocprofv3 --pmc {LDS_COUNTERS} --kernel-trace -d <outdir> -o run -f csv -- "
         f"python3 bench.py {PMC_ARGS}\n```\n",
         "Per dispatch, averaged over each kernel's dispatches. SIMD cycles = GRBM_GUI_ACTIVE / "
         f"{N_XCD} x {N_CU} CUs x {SIMD_PER_CU}. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD cycles; "
         "VALU issuing = 4 x SQ_ACTIVE_INST_VALU (quad-cycles) / SIMD cycles; both = "
         "SQ_VALU_MFMA_COEXEC_CYCLES / SIMD cycles (a VALU instruction running beside an MFMA); "
         "waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES (share of a wave's life at a wait count or a "
         "barrier), not issuing = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; VALU / MFMA = SQ_INSTS_VALU / "
         "SQ_INSTS_MFMA (the VALU count includes the MFMAs); LDS read B/clk per CU = 64 x "
         "SQ_INSTS_LDS_LOAD_BANDWIDTH / CU cycles; bank-conflict share = SQ_LDS_BANK_CONFLICT / "
         "SQ_LDS_IDX_ACTIVE; LDS wait per LDS instruction = SQ_WAIT_INST_LDS / "
         "SQ_ACTIVE_INST_LDS.\n",
         "| kernel | role | MFMA busy | VALU issuing | both | waiting | not issuing | VALU / MFMA | "
         "LDS read B/clk/CU | bank-conflict share | LDS wait per LDS inst |",
         "|---|---|---|---|---|---|---|---|---|---|---|"]
    for n in cols["mfma"]:
        g = lambda k: cols[k].get(n, float("nan"))
        L.append(f"| `{short_name(n)}` | {role(n)} | {100 * g('mfma'):.1f}% | {100 * g('valu'):.1f}% | "
                 f"{100 * g('coexec'):.1f}% | {100 * g('wait'):.1f}% | {100 * g('waitinst'):.1f}% | "
                 f"{'-' if g('vpm') != g('vpm') else format(g('vpm'), '.2f')} | {g('ldsbw'):.1f} | {100 * g('conf'):.1f}% | {g('ldswait'):.2f} |")
    open(os.path.join(out, f"attn_{bench['dtype']}_{bench['config']['workload']}_pipeline.md"), "w").write(
        "\n".join(L) + "\n")


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
         "then 1 + 3 steps of the three-call path (reorder q, k, v; tile-major STA; restore), "
         "1 + 2 dense-comparator launches, 1 + 3 forward-with-lse and backward passes at the same "
         "shape, 1 + 2 window-recall passes, 1 + 3 launches of the fp8 q/k forward, then 1 + 3 "
         "launches on each other named workload (the same kernels).\n",
         "| kernel | role | calls | average (ms) | min (ms) | max (ms) | share |",
         "|---|---|---|---|---|---|---|"]
    for r in rows:
        L.append(f"| `{short_name(r['Name'])}` | {role(r['Name'])} | {r['Calls']} | "
                 f"{float(r['AverageNs']) / 1e6:.3f} | {float(r['MinNs']) / 1e6:.3f} | "
                 f"{float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.1f}% |")
    rf = bench["roofline"]
    # The same kernel also serves the backward's forward and the other
    # workloads later in the run, so the --stats average mixes shapes; the
    # timed launches are the first warmup + steps dispatches of the kernel.
    timed = None
    tpath = os.path.join(run, "trace", "bench_kernel_trace.csv")
    if os.path.exists(tpath):
        fused = cfg.get("path", "fused") == "fused"
        rows_t = list(csv.DictReader(open(tpath)))
        dur = {int(r["Dispatch_Id"]): int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows_t}
        if fused:
            steps = step_dispatches((int(r["Dispatch_Id"]), r["Kernel_Name"]) for r in rows_t)
        else:
            steps = sorted((int(r["Dispatch_Id"]), None) for r in rows_t
                           if role(r["Kernel_Name"]) == "STA forward, tile-major (three-call path)")
        w0, ns = bench["warmup"], bench["steps"]
        if len(steps) >= w0 + ns:
            sel = steps[w0:w0 + ns]
            main_ms = sum(dur[m] for m, _ in sel) / len(sel) / 1e6
            tail_ms = sum(dur[t] for _, t in sel if t is not None) / len(sel) / 1e6
            timed = (main_ms, tail_ms, sum(1 for _, t in sel if t is not None))
    if timed is None:
        tline = "n/a (no kernel trace)."
    elif timed[2]:
        tline = (f"{timed[0]:.3f} ms (whole-tile items) + {timed[1]:.3f} ms (the last round as 64-row "
                 f"items, a second launch) = {timed[0] + timed[1]:.3f} ms a step in the trace.")
    else:
        tline = f"{timed[0]:.3f} ms in the trace."
    L += ["", f"Timed steps: steps {bench['warmup'] + 1}..{bench['warmup'] + bench['steps']} of "
          f"the {rf['kernel']} (the first warm-up + timed steps of that path in the run) average "
          + tline,
          f"bench.py's HIP-event average for the same launches in the same command without the "
          f"profiler: {rf['launch_ms']:.3f} ms, {rf['achieved']:.1f} TFLOP/s of algorithmic work "
          f"({cfg['algorithmic_tflop_per_step']:.4f} TFLOP per launch), {100 * rf['frac']:.1f}% of "
          f"the {rf['peak']:.0f} TFLOP/s dense peak."]
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
    # headline: the fused kernel's first 1 + 2 dispatches (warm-up + timed
    # steps of the counter runs); later dispatches of the same kernel belong
    # to other workloads
    # a step's traffic: its whole-tile launch plus its tail launch, if any
    names = {d: n for (d, n) in fetch}
    hsteps = step_dispatches(names.items())[:3]
    head = [(m, names[m]) for m, _ in hsteps]
    if head:
        def per_step(c):
            return sum(c.get((m, names[m]), 0.0) + (c.get((t, names[t]), 0.0) if t is not None else 0.0)
                       for m, t in hsteps) / len(hsteps)
        hf, hw = per_step(fetch), per_step(write)
        records["fused"] = {
            "kernel": short_name(head[0][1]), "workload": wl, "path": "fused",
            "dispatches": len(head),
            "source_sha256": source_sha256(),
            "read_bytes_per_launch": hf * fscale * 1024,
            "write_bytes_per_launch": hw * wscale * 1024,
            "bytes_per_launch": hf * fscale * 1024 + hw * wscale * 1024,
            "algorithmic_bytes_per_launch": 4 * tensor,
            "fetch_kib_to_bytes": fscale * 1024, "write_kib_to_bytes": wscale * 1024,
            "commands": [pmc_cmd("FETCH_SIZE"), pmc_cmd("WRITE_SIZE")],
        }
        L.append(f"| `{short_name(head[0][1])}` | the timed steps of the fused path only (with their "
                 f"64-row tail launches) | {len(head)} | "
                 f"{hf:.0f} | {hw:.0f} | {hf * fscale * 1024 / 1e9:.3f} | {hw * wscale * 1024 / 1e9:.3f} | "
                 f"{3 * tensor / 1e9:.3f} + {tensor / 1e9:.3f} |")
    for n in kernels:
        f, w, c = summarize(lambda x, n=n: x == n)
        r = role(n)
        if "reorder" in n:
            alg = f"{tensor / 1e9:.3f} + {tensor / 1e9:.3f}"
        elif r.endswith("fp8 q and k"):   # q and k at one byte an element
            alg = f"{2 * tensor / 1e9:.3f} + {tensor / 1e9:.3f}"
        elif r.startswith(("STA forward, raster", "STA forward, tile-major", "dense comparator")) and "only" not in r:
            alg = f"{3 * tensor / 1e9:.3f} + {tensor / 1e9:.3f}"
        else:
            alg = "-"
        L.append(f"| `{short_name(n)}` | {role(n)} | {c} | {f:.0f} | {w:.0f} | "
                 f"{f * fscale * 1024 / 1e9:.3f} | {w * wscale * 1024 / 1e9:.3f} | {alg} |")
        path = "three_call" if role(n) == "STA forward, tile-major (three-call path)" else None
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
    # the tile-major path's step: add its 64-row tail launch, if it has one
    tails = [n for n in kernels if role(n).startswith("STA forward, tile-major (three-call path), 64-row items")]
    if "three_call" in records and tails:
        f, w, _ = summarize(lambda x: x == tails[0])
        rec = records["three_call"]
        rec["read_bytes_per_launch"] += f * fscale * 1024
        rec["write_bytes_per_launch"] += w * wscale * 1024
        rec["bytes_per_launch"] = rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
        rec["tail_kernel"] = short_name(tails[0])
    if "fused" in records and any(t is not None for _, t in hsteps):
        rec = records["fused"]
        rec["tail_kernel"] = short_name(names[next(t for _, t in hsteps if t is not None)])
    L += ["", "\"Algorithmic\" counts every input element once and every output element once "
          "(q, k, v read; o written). The attention kernels re-read K and V for every query tile "
          "whose window holds them; what the counters show is the traffic below L2 (HBM and the "
          "memory-side cache). A step of either path is one launch of whole-tile items and, when "
          "the items do not fill the last round, a second launch of that round as 64-row items; "
          "the JSON records count both."]
    open(os.path.join(out, f"attn_{bench['dtype']}_{wl}_traffic.md"), "w").write("\n".join(L) + "\n")
    for path, rec in records.items():
        fn = os.path.join(out, f"attn_{bench['dtype']}_{path}_{wl}_traffic.json")
        json.dump(rec, open(fn, "w"), indent=1)

    # MFMA busy fraction.
    mpath = os.path.join(run, "MFMA", "run_counter_collection.csv")
    if os.path.exists(mpath):
        busy = per_dispatch(mpath, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui = per_dispatch(mpath, "GRBM_GUI_ACTIVE")
        sq = per_dispatch(mpath, "SQ_BUSY_CYCLES")
        L = [f"# Matrix-core busy fraction, bench.py on {title}\n",
             "Command (repo root), one pass:\n",
             f"```\nrocprofv3 --pmc {MFMA_COUNTERS} --kernel-trace -d <outdir> -o run -f csv -- "
             f"python3 bench.py {PMC_ARGS}\n```\n",
             f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCD} x {N_CU} CUs x "
             f"{SIMD_PER_CU} SIMDs), per dispatch, averaged over the dispatches of each kernel "
             f"(rocprofv3 reports GRBM_GUI_ACTIVE summed over the {N_XCD} XCDs, and "
             "SQ_VALU_MFMA_BUSY_CYCLES summed over all SIMDs: 16 per 16x16x32 bf16 MFMA). "
             "GRBM_GUI_ACTIVE counts the cycles of the dispatch at the clock the chip ran, so "
             "the ratio is the matrix cores' duty cycle; 'clock' is the one implied by "
             "GRBM_GUI_ACTIVE and the dispatch time.\n",
             "| kernel | role | dispatches | MFMA busy | clock (GHz) |",
             "|---|---|---|---|---|"]
        dur = {}
        for r in csv.DictReader(open(mpath)):
            dur[(int(r["Dispatch_Id"]), r["Kernel_Name"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        names = list(dict.fromkeys(n for (_, n) in busy if role(n)))
        for n in names:
            ks = [k for k in busy if k[1] == n and gui.get(k)]
            if not ks:
                continue
            fr = [busy[k] / (gui[k] / N_XCD * N_CU * SIMD_PER_CU) for k in ks]
            clk = [gui[k] / N_XCD / dur[k] for k in ks if dur.get(k)]
            L.append(f"| `{short_name(n)}` | {role(n)} | {len(fr)} | {100 * sum(fr) / len(fr):.1f}% | "
                     f"{(sum(clk) / len(clk)) if clk else float('nan'):.2f} |")
        open(os.path.join(out, f"attn_{bench['dtype']}_{wl}_mfma_busy.md"), "w").write("\n".join(L) + "\n")
    pipeline_summary(run, out, bench, title)
    print(json.dumps({p: r["bytes_per_launch"] for p, r in records.items()}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
