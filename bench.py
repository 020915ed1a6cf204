#!/usr/bin/env python3
"""Benchmark of the Sliding Tile Attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch of synthetic raster-
order input already resident in HBM. By default (--path fused) that is one
sta_forward_raster launch: the tile grouping of queries and keys, the window
enumeration and the flash loop in one kernel. --path three_call times
sta_reorder_tiles on q, k and v, sta_forward and sta_restore_order instead.
The headline value is effective TFLOP/s over the step, counting only computed
blocks: 4 * tau^2 * head_dim FLOPs per (query tile, key tile) pair.

Printed as one JSON line. Besides the contract fields it carries
  roofline      the attention kernel (dominant) against the bf16 MFMA peak,
                timed with HIP events on the stream it runs on;
  cpu_baseline  the CPU oracle timed on a bounded sample of the workload;
  dense         the dense comparator at the same shape and the speed-up;
  three_call    the reorder -> tile-major forward -> restore path, with the
                permutation kernels' achieved HBM bandwidth;
  backward      sta_forward_lse + sta_backward at the same shape;
  recall        sta_window_recall over five candidate windows at the same shape;
  fp8_qk        sta_forward_fp8 (e4m3 q and k, bf16 v) at the same shape, against
                the mixed peak of its two products (QK^T at the fp8 MFMA peak,
                PV at the bf16 one);
  other_workloads  the fused kernel on the other named workloads (and, on the
                small float32 one, sta_backward).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
# Half the counted work (QK^T) at the fp8 peak, half (PV) at the bf16 peak.
FP8_QK_PEAK_TFLOPS = 1.0 / (0.5 / FP8_PEAK_TFLOPS + 0.5 / BF16_PEAK_TFLOPS)
F32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector, published
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "STA fwd effective TFLOP/s + MFMA util, 30x48x80 latent, w=(18,24,24), 1 GPU"


def algorithmic_flops(w, windows) -> float:
    """4 * tau^2 * d per computed (query tile, key tile) pair, times B."""
    from sparse_attention_video_tile_amd import binding
    pairs = binding.sta_kv_pair_count(w.heads, w.volume, w.tile, windows)
    tau = w.tile[0] * w.tile[1] * w.tile[2]
    return float(w.B) * pairs * 4.0 * tau * tau * w.head_dim


def gpu_inputs(w, torch):
    """Seeded N(0,1) tensors of the workload's shape drawn on the device."""
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    shape = (w.B, w.heads) + tuple(w.volume) + (w.head_dim,)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return [torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dt) for _ in range(3)]


def recorded_traffic(workload: str, path_name: str):
    """HBM-side bytes per attention launch from the committed counter record
    (profiles/), or None when there is none for this workload and path or the
    kernel sources' code (comments aside) has changed since the counters were
    taken."""
    from sparse_attention_video_tile_amd.profile_summary import source_sha256
    path = os.path.join(ROOT, "profiles", f"attn_bf16_{path_name}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_sha256(ROOT):
        return None
    return float(rec["bytes_per_launch"])


def cpu_baseline(w, whole_head: bool = True):
    """The oracle as it stands, timed on the host's cores: a process pool of
    (batch, head, query tile) jobs, one BLAS thread per worker, over
    os.sched_getaffinity(0) cores (at most 16, one GPU's share of the box).
    Times the tiny fp32 workload whole, then one whole head of the benchmarked
    workload (a one-head draw of its shape and window: all its query tiles),
    or 32 query tiles of it with whole_head=False. The oracle's cost per query
    tile does not depend on the window (it scores every key and masks), so
    each 30x48x80 workload extrapolates to heads x the one-head time."""
    import oracle
    from oracle import pool
    from sparse_attention_video_tile_amd import workloads
    scale = 1.0 / math.sqrt(w.head_dim)
    tiny = workloads.TINY_F32
    ti = workloads.make_inputs(tiny)
    _, tiny_s, _ = pool.sta_attention_pool(
        ti.q, ti.k, ti.v, tiny.tile, ti.windows, 1.0 / math.sqrt(tiny.head_dim),
        pool.tile_jobs(tiny.volume, tiny.tile, [(0, h) for h in range(tiny.heads)]))
    one = w.with_(heads=1, windows=None if w.windows is None else w.windows[:1])
    inp = workloads.make_inputs(one)
    n = oracle.tile_grid(w.volume, w.tile)
    n_tiles = n[0] * n[1] * n[2]
    tiles = range(n_tiles) if whole_head else range(0, n_tiles, max(1, n_tiles // 32))
    jobs = pool.tile_jobs(w.volume, w.tile, [(0, 0)], tiles)
    _, wall, workers = pool.sta_attention_pool(inp.q, inp.k, inp.v, w.tile, inp.windows, scale, jobs)
    window = tuple(int(x) for x in inp.windows[0])
    om = oracle.window_in_tiles(window, w.tile, w.volume)
    tau = w.tile[0] * w.tile[1] * w.tile[2]
    flops = len(jobs) * om[0] * om[1] * om[2] * 4.0 * tau * tau * w.head_dim
    per_head_s = wall * n_tiles / len(jobs)
    return {
        "value": flops / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": int(workers),
        "kind": "oracle",
        "sample": f"{len(jobs)} query tiles ({len(jobs) * tau} rows) of one head, window {window}, "
                  f"of a one-head draw of {w.name}: {wall:.1f} s on a pool of {workers} "
                  f"single-thread workers; {tiny.name} whole ({tiny.heads} heads): {tiny_s:.1f} s",
        "wall_s": wall,
        "tiny_f32_whole_s": tiny_s,
        "one_head_s": per_head_s,
        "extrapolated_workload_s": per_head_s * w.heads * w.B,
        "extrapolation": "oracle cost per query tile is window-independent: every 30x48x80 "
                         "workload (all windows) takes heads x one_head_s",
    }


def time_backward(w, args, torch, binding, q, k, v, windows, fwd_flops, stream, ev):
    """sta_forward_lse + sta_backward (raster order) on the headline inputs with
    a seeded N(0,1) upstream gradient. TFLOP/s count the five products of the
    usual attention backward (QK^T, dO V^T, P^T dO, dS^T Q, dS K: 2.5 x the
    forward's FLOPs); the kernels issue seven (QK^T and dO V^T are recomputed
    on both the key side and the query side), reported as mfma_tflops."""
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 1000)
    dout = torch.randn(q.shape, generator=g, device="cuda", dtype=torch.float32).to(q.dtype)
    out, lse = binding.sta_forward_lse(q, k, v, w.tile, windows)
    delta = torch.empty_like(lse)
    binding.sta_backward(q, k, v, out, dout, lse, w.tile, windows, delta=delta)  # warm-up
    torch.cuda.synchronize()
    e0, e1, e2 = ev(), ev(), ev()
    e0.record(stream)
    for _ in range(args.backward_reps):
        binding.sta_forward_lse(q, k, v, w.tile, windows, out=out, lse=lse)
    e1.record(stream)
    for _ in range(args.backward_reps):
        grads = binding.sta_backward(q, k, v, out, dout, lse, w.tile, windows, delta=delta)
    e2.record(stream)
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / args.backward_reps
    bwd_ms = e1.elapsed_time(e2) / args.backward_reps
    bwd_flops = 2.5 * fwd_flops
    del grads, dout, out, lse, delta
    return {
        "forward_lse_ms": fwd_ms,
        "backward_ms": bwd_ms,
        "backward_tflops": bwd_flops / (bwd_ms * 1e-3) / 1e12,
        "backward_frac_of_peak": bwd_flops / (bwd_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "backward_mfma_tflops": 3.5 * fwd_flops / (bwd_ms * 1e-3) / 1e12,
        "algorithmic_tflop": bwd_flops / 1e12,
        "train_step_ms": fwd_ms + bwd_ms,
        "train_step_tflops": (fwd_flops + bwd_flops) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12,
        "order": "raster",
    }


def time_recall(w, args, torch, binding, workloads, q, k, stream, ev):
    """sta_window_recall over the five window options of the mixed workload
    on the headline q, k. Work counted: the QK^T products of the full-attention
    log-sum-exp (2 S^2 d per head), which every candidate's sums come out of
    (one pass; separate candidate passes would add 2 tau^2 d per computed tile
    pair of each window); the exponentials are not counted."""
    cands = [tuple(c) for c in workloads.MIXED_WINDOW_OPTIONS]
    S = w.seq_len
    tau = w.tile[0] * w.tile[1] * w.tile[2]
    flops = float(w.B) * w.heads * 2.0 * S * S * w.head_dim
    per_candidate = sum(float(w.B) * binding.sta_kv_pair_count(w.heads, w.volume, w.tile, [c]) * 2.0 * tau * tau
                        * w.head_dim for c in cands)
    ws = torch.empty((len(cands) + 1, w.B, w.heads, S), dtype=torch.float32, device="cuda")
    r = binding.sta_window_recall(q, k, w.tile, cands, workspace=ws)  # warm-up
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(args.recall_reps):
        r = binding.sta_window_recall(q, k, w.tile, cands, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.recall_reps
    tf = flops / (ms * 1e-3) / 1e12
    mean = r.mean(dim=(0, 1)).cpu().tolist()
    del ws, r
    return {"ms": ms, "tflops": tf, "frac_of_peak": tf / BF16_PEAK_TFLOPS, "algorithmic_tflop": flops / 1e12,
            "candidate_passes_tflop": per_candidate / 1e12,
            "candidates": cands, "mean_recall_on_iid_inputs": mean}


def time_fp8(w, args, torch, binding, q, k, v, out, windows, flops, stream, ev):
    """sta_forward_fp8 on the headline raster tensors: q and k quantized to
    e4m3 with power-of-two per-tensor descales before the timed region."""
    codes = []
    for x in (q, k):
        amax = float(x.float().abs().max())
        descale = 2.0 ** math.ceil(math.log2(max(amax, 1e-30) / 448.0))
        codes.append(((x.float() / descale).to(torch.float8_e4m3fn).view(torch.uint8), descale))
    (q8, qd), (k8, kd) = codes
    binding.sta_forward_fp8(q8, k8, v, w.tile, windows, qd, kd, out=out)  # warm-up
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(args.fp8_reps):
        binding.sta_forward_fp8(q8, k8, v, w.tile, windows, qd, kd, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.fp8_reps
    tf = flops / (ms * 1e-3) / 1e12
    del q8, k8
    return {"ms": ms, "tflops": tf, "peak": FP8_QK_PEAK_TFLOPS, "frac_of_peak": tf / FP8_QK_PEAK_TFLOPS,
            "frac_of_bf16_peak": tf / BF16_PEAK_TFLOPS, "kernel": "attn_bf16_kernel, QK8 (raster order)"}


def other_workloads(main_w, args, torch, binding, workloads, q, k, v, out, stream, ev):
    """The fused kernel on every other named workload: average launch time,
    effective TFLOP/s and fraction of peak. Workloads of the headline shape
    reuse its device tensors (timing does not depend on the values)."""
    res = {}
    for w in workloads.NAMED:
        if w.name == main_w.name:
            continue
        windows = workloads.head_windows(w)
        flops = algorithmic_flops(w, windows)
        same = (w.B, w.heads, w.head_dim, tuple(w.volume), w.dtype) == \
            (main_w.B, main_w.heads, main_w.head_dim, tuple(main_w.volume), main_w.dtype)
        if same:
            a, b, c, o = q, k, v, out
        else:
            a, b, c = gpu_inputs(w, torch)
            o = torch.empty_like(a)
        try:
            binding.sta_forward_raster(a, b, c, w.tile, windows, out=o)  # warm-up
        except NotImplementedError:   # no raster-order kernel for this workload
            continue
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.config_reps):
            binding.sta_forward_raster(a, b, c, w.tile, windows, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.config_reps
        tf = flops / (ms * 1e-3) / 1e12
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
        res[w.name] = {"ms": ms, "tflops": tf, "frac_of_peak": tf / peak, "dtype": w.dtype,
                       "algorithmic_tflop": flops / 1e12,
                       "windows": sorted({tuple(x) for x in windows.tolist()})}
        if not same:
            # the small workloads also time their backward (five-product count)
            dout = torch.randn(a.shape, device="cuda", dtype=torch.float32).to(a.dtype)
            o, lse = binding.sta_forward_lse(a, b, c, w.tile, windows)
            delta = torch.empty_like(lse)
            binding.sta_backward(a, b, c, o, dout, lse, w.tile, windows, delta=delta)  # warm-up
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(args.config_reps):
                binding.sta_backward(a, b, c, o, dout, lse, w.tile, windows, delta=delta)
            e1.record(stream)
            torch.cuda.synchronize()
            bms = e0.elapsed_time(e1) / args.config_reps
            res[w.name].update({"backward_ms": bms,
                                "backward_frac_of_peak": 2.5 * flops / (bms * 1e-3) / 1e12 / peak})
            del a, b, c, o, dout, lse, delta
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sta_30x48x80_w18x24x24")
    ap.add_argument("--path", choices=("fused", "three_call"), default="fused",
                    help="fused: one raster-order kernel; three_call: reorder, forward, restore")
    ap.add_argument("--compare-reps", type=int, default=3,
                    help="steps of the other path to time for comparison (0: skip)")
    ap.add_argument("--dense-reps", type=int, default=2, help="dense comparator launches to time (0: skip)")
    ap.add_argument("--cpu", choices=("head", "sample", "none"), default="head",
                    help="CPU oracle baseline: one whole head (default), 32 query tiles, or skip")
    ap.add_argument("--backward-reps", type=int, default=3,
                    help="STA backward launches to time at the headline workload (0: skip)")
    ap.add_argument("--recall-reps", type=int, default=2,
                    help="window-recall scoring runs to time at the headline shape (0: skip)")
    ap.add_argument("--fp8-reps", type=int, default=3,
                    help="sta_forward_fp8 launches to time (0: skip)")
    ap.add_argument("--config-reps", type=int, default=3,
                    help="launches per other named workload to time (0: skip)")
    ap.add_argument("--copy-reference", action="store_true",
                    help="run one plain device copy of a q-sized tensor first (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the STA path is built and timed on a single "
              "MI355X; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from sparse_attention_video_tile_amd import binding, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    binding.load_library()
    w = workloads.by_name(args.workload)
    windows = workloads.head_windows(w)
    flops = algorithmic_flops(w, windows)
    S = w.seq_len
    q, k, v = gpu_inputs(w, torch)
    qt, kt, vt = (torch.empty((w.B, w.heads, S, w.head_dim), dtype=q.dtype, device="cuda") for _ in range(3))
    ot = torch.empty_like(qt)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    fused = args.path == "fused"
    if fused:
        try:
            binding.sta_forward_raster(q, k, v, w.tile, windows, out=out)
        except NotImplementedError as e:
            print(f"{w.name}: no raster-order kernel ({e}); use --path three_call", file=sys.stderr)
            return 2

    def step_fused(timers=None):
        if timers is not None:
            timers[0].record(stream)
        binding.sta_forward_raster(q, k, v, w.tile, windows, out=out)
        if timers is not None:
            timers[1].record(stream)

    def step_three(timers=None):
        if timers is not None:
            timers[0].record(stream)
        for src, dst in ((q, qt), (k, kt), (v, vt)):
            binding.sta_reorder_tiles(src, w.tile, out=dst)
        if timers is not None:
            timers[1].record(stream)
        binding.sta_forward(qt, kt, vt, w.volume, w.tile, windows, out=ot)
        if timers is not None:
            timers[2].record(stream)
        binding.sta_restore_order(ot, w.volume, w.tile, out=out)
        if timers is not None:
            timers[3].record(stream)

    def timed(step, n_steps, n_events):
        timers = [[ev() for _ in range(n_events)] for _ in range(n_steps)]
        start, stop = ev(), ev()
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(n_steps):
            step(timers[i])
        stop.record(stream)
        torch.cuda.synchronize()
        spans = [float(np.mean([t[j].elapsed_time(t[j + 1]) for t in timers]))
                 for j in range(n_events - 1)]
        return start.elapsed_time(stop) / n_steps, spans

    step = step_fused if fused else step_three
    if args.copy_reference:
        out.copy_(q)  # a plain copy kernel: reads and writes exactly one tensor
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_per_step, spans = timed(step, args.steps, 2 if fused else 4)
    attn_ms = spans[0] if fused else spans[1]
    elem = 2 if w.dtype == "bf16" else 4
    tensor_bytes = w.B * w.heads * S * w.head_dim * elem
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12

    three = None
    if not fused or args.compare_reps > 0:
        if fused:
            step_three()
            three_ms, tspans = timed(step_three, args.compare_reps, 4)
        else:
            three_ms, tspans = ms_per_step, spans
        reorder_ms, fwd_ms, restore_ms = tspans
        three = {
            "ms": three_ms,
            "tflops": flops / (three_ms * 1e-3) / 1e12,
            "forward_ms": fwd_ms,
            "reorder_qkv_ms": reorder_ms,
            "reorder_qkv_gbs": 3 * 2 * tensor_bytes / (reorder_ms * 1e-3) / 1e9,
            "restore_ms": restore_ms,
            "restore_gbs": 2 * tensor_bytes / (restore_ms * 1e-3) / 1e9,
            "hbm_peak_gbs": HBM_PEAK_GBS,
        }

    dense = None
    if args.dense_reps > 0:
        qd, kd, vd = (x.view(w.B, w.heads, S, w.head_dim) for x in (q, k, v))
        od = torch.empty_like(qd)
        binding.sta_full_attention(qd, kd, vd, out=od)  # warm-up
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(args.dense_reps):
            binding.sta_full_attention(qd, kd, vd, out=od)
        b.record(stream)
        torch.cuda.synchronize()
        dense_ms = a.elapsed_time(b) / args.dense_reps
        dense_flops = float(w.B) * w.heads * 4.0 * S * S * w.head_dim
        dense = {"ms": dense_ms, "tflops": dense_flops / (dense_ms * 1e-3) / 1e12,
                 "speedup_sta_vs_dense": dense_ms / attn_ms}
        del qd, kd, vd, od

    backward = None
    if args.backward_reps > 0 and fused:
        backward = time_backward(w, args, torch, binding, q, k, v, windows, flops, stream, ev)

    recall = None
    if args.recall_reps > 0 and fused:
        recall = time_recall(w, args, torch, binding, workloads, q, k, stream, ev)

    fp8 = None
    if args.fp8_reps > 0 and fused and w.dtype == "bf16" and w.head_dim == 128:
        fp8 = time_fp8(w, args, torch, binding, q, k, v, out, windows, flops, stream, ev)

    others = None
    if args.config_reps > 0:
        others = other_workloads(w, args, torch, binding, workloads, q, k, v, out, stream, ev)

    cpu = cpu_baseline(w, whole_head=args.cpu == "head") if args.cpu != "none" else None

    result = {
        "metric": METRIC,
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": w.B, "heads": w.heads, "head_dim": w.head_dim,
            "volume": list(w.volume), "tile": list(w.tile),
            "windows": sorted({tuple(x) for x in windows.tolist()}),
            "path": args.path,
            "algorithmic_tflop_per_step": flops / 1e12,
            "inputs": "seeded N(0,1) q, k, v drawn on the device, rounded to bf16",
        },
        "roofline": {
            "kernel": ("attn_bf16_kernel" if w.dtype == "bf16" else "attn_f32_kernel")
                      + (" (raster order)" if fused else " (tile-major order)"),
            "bound": "mfma",
            "achieved": attn_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": attn_tflops / peak,
            "traffic": recorded_traffic(w.name, args.path) if w.dtype == "bf16" else None,
            "launch_ms": attn_ms,
            "launch_note": "one step's attention launches, HIP events around them: whole-tile work "
                           "items, then (when they leave the last round mostly idle) that round "
                           "as 64-row items (keys split over two wave groups) in a second launch",
        },
        "cpu_baseline": cpu,
        "dense": dense,
        "three_call": three,
        "backward": backward,
        "recall": recall,
        "fp8_qk": fp8,
        "other_workloads": others,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
