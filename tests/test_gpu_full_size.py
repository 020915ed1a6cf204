"""GPU: the four 30x48x80 workloads at full size, in the launch configuration
the benchmark times (the raster-order kernel). The oracle computes sampled
query rows one by one (corner, edge and interior tiles of several heads), and
every row of one whole head of the (18,24,24) workload and of the mixed
workload's heaviest head that is not the whole volume, and the last four
tiles of every head (a process pool of the oracle over the host's cores);
whole-volume STA is also compared element by element with the dense kernel,
and the raster-order kernel with the reorder + tile-major path; and a padded
grid of the same tile grid, whose last round runs with every odd key chunk
padding only."""

import time

import numpy as np
import pytest
import torch

import oracle
from oracle import pool
from sparse_attention_video_tile_amd import binding, workloads
from tests.parity_util import assert_close, default_scale, to_gpu

pytestmark = pytest.mark.gpu

FULL = [workloads.STA_18_24_24, workloads.STA_30_40_40, workloads.DENSE_WHOLE, workloads.MIXED_HEADS]


def sample_rows(w, windows, rng):
    """(head, raster query tokens) samples: corner / edge / interior tiles."""
    n = oracle.tile_grid(w.volume, w.tile)
    n_tiles = n[0] * n[1] * n[2]
    heads = {0, w.heads - 1, int(rng.integers(0, w.heads))}
    for opt in {tuple(x) for x in windows.tolist()}:  # one head per distinct window
        heads.add(int(np.nonzero((windows == opt).all(axis=1))[0][0]))
    interior = ((n[0] // 2) * n[1] + n[1] // 2) * n[2] + n[2] // 2
    edge = ((0 * n[1]) + n[1] - 1) * n[2] + n[2] // 2
    tiles = sorted({0, n_tiles - 1, interior, edge, int(rng.integers(0, n_tiles))})
    out = []
    for h in sorted(heads):
        rows = []
        for t in tiles:
            toks = oracle.tile_tokens(w.volume, w.tile, t)
            pick = np.unique(np.concatenate([toks[[0, -1]], rng.choice(toks, 6, replace=False)]))
            rows.append(pick)
        out.append((h, np.concatenate(rows)))
    return out


def whole_head(w, windows) -> int:
    """Head checked row by row: head 0 of a uniform workload; of the mixed one,
    the head with the largest window that is not the whole volume."""
    if w.windows is not None:
        return 0
    sizes = [int(np.prod(x)) for x in windows]
    full = int(np.prod(w.volume))
    return max((i for i in range(len(sizes)) if sizes[i] < full), key=lambda i: (sizes[i], -i))


@pytest.mark.timeout(400)   # input draws, then up to a whole head of the oracle on the host
@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_full_size_sampled_rows(w):
    print(f"[case] full size {w.name}: generating inputs", flush=True)
    inp = workloads.make_inputs(w)
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    print(f"[case] full size {w.name}: running the path", flush=True)
    out = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().reshape(w.B, w.heads, -1, w.head_dim)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(w.seed)
    scale = default_scale(w.head_dim)
    gots, refs = [], []
    for h, rows in sample_rows(w, inp.windows, rng):
        window = tuple(int(x) for x in inp.windows[h])
        ref = oracle.sta_attention_rows(inp.q, inp.k, inp.v, w.tile, window, scale, 0, h, rows)
        gots.append(got[0, h, rows])
        refs.append(ref)
        assert_close(got[0, h, rows], ref, w.dtype, f"{w.name} head {h} window {window}")
    assert_close(np.concatenate(gots), np.concatenate(refs), w.dtype, f"{w.name} all samples")

    if w is workloads.STA_18_24_24 or w is workloads.MIXED_HEADS:
        h = whole_head(w, inp.windows)
        window = tuple(int(x) for x in inp.windows[h])
        print(f"[case] full size {w.name}: every row of head {h}, window {window}, oracle pool",
              flush=True)
        last = [time.perf_counter()]

        def progress(done, total):
            if time.perf_counter() - last[0] > 10 or done == total:
                last[0] = time.perf_counter()
                print(f"[oracle] {done}/{total} query tiles", flush=True)

        jobs = pool.tile_jobs(w.volume, w.tile, [(0, h)])
        ref, wall, workers = pool.sta_attention_pool(inp.q, inp.k, inp.v, w.tile, inp.windows, scale,
                                                     jobs, progress=progress)
        print(f"[oracle] head {h}: {wall:.1f} s on {workers} workers", flush=True)
        assert_close(got[0, h], ref[(0, h)], w.dtype, f"{w.name} head {h} all {w.seq_len} rows")

    if w is workloads.DENSE_WHOLE:
        print(f"[case] full size {w.name}: dense kernel", flush=True)
        S = w.seq_len
        dense = binding.sta_full_attention(q.view(w.B, w.heads, S, w.head_dim),
                                           k.view(w.B, w.heads, S, w.head_dim),
                                           v.view(w.B, w.heads, S, w.head_dim))
        diff = (dense.float() - out.view(w.B, w.heads, S, w.head_dim).float()).abs()
        print(f"[parity] whole-volume STA vs dense: max {diff.max().item():.3e} "
              f"mean {diff.mean().item():.3e}", flush=True)
        assert diff.max().item() <= 2e-2 and diff.mean().item() <= 2e-3


@pytest.mark.timeout(300)   # input draws, then 96 query tiles of the oracle on the host
def test_full_size_last_tiles_of_every_head():
    """Every row of the last four query tiles of every head of the (18,24,24)
    workload: at 24 heads the 7200 whole-tile work items leave a partly filled
    last round on each XCD, which runs as 64-row items in a second launch, and
    those items are last tiles of heads. Checked against the oracle (process
    pool) element by element."""
    w = workloads.STA_18_24_24
    print(f"[case] full size {w.name}: last four tiles of every head", flush=True)
    inp = workloads.make_inputs(w)
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    out = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().reshape(w.B, w.heads, -1, w.head_dim)
    n = oracle.tile_grid(w.volume, w.tile)
    n_tiles = n[0] * n[1] * n[2]
    last = list(range(n_tiles - 4, n_tiles))
    jobs = pool.tile_jobs(w.volume, w.tile, [(0, h) for h in range(w.heads)], tiles=last)
    ref, wall, workers = pool.sta_attention_pool(inp.q, inp.k, inp.v, w.tile, inp.windows,
                                                 default_scale(w.head_dim), jobs)
    print(f"[oracle] {len(jobs)} tiles: {wall:.1f} s on {workers} workers", flush=True)
    for h in range(w.heads):
        rows = np.concatenate([oracle.tile_tokens(w.volume, w.tile, t) for t in last])
        assert_close(got[0, h, rows], ref[(0, h)][rows], w.dtype, f"{w.name} head {h} last tiles")


@pytest.mark.timeout(300)   # input draws, then 96 query tiles of the oracle on the host
def test_padded_full_size_last_tiles_of_every_head():
    """A padded grid at full size: 25x47x79 with (6,8,8) tiles is the 5x6x10
    tile grid of the named workloads, its last t-tile holding one plane of
    tokens. At 24 heads the last round again runs as 64-row items whose two
    wave groups take the even and the odd key chunks; with window (6,24,24)
    the last tiles' windows lie in that one-plane t-tile, so every odd chunk
    (and the odd group's first) holds padding only. Every row of the last four
    tiles of every head against the oracle, and the raster kernel against the
    reorder + tile-major path bit for bit."""
    w = workloads.small_case((25, 47, 79), (6, 8, 8), [(6, 24, 24)] * 24, seed=11,
                             name="padded_25x47x79_w6x24x24")
    print(f"[case] full size {w.name}: last four tiles of every head", flush=True)
    inp = workloads.make_inputs(w)
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    out = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows, fused=True)
    alt = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(out, alt)
    got = out.float().cpu().numpy().reshape(w.B, w.heads, -1, w.head_dim)
    assert np.isfinite(got).all()
    n = oracle.tile_grid(w.volume, w.tile)
    n_tiles = n[0] * n[1] * n[2]
    last = list(range(n_tiles - 4, n_tiles))
    jobs = pool.tile_jobs(w.volume, w.tile, [(0, h) for h in range(w.heads)], tiles=last)
    ref, wall, workers = pool.sta_attention_pool(inp.q, inp.k, inp.v, w.tile, inp.windows,
                                                 default_scale(w.head_dim), jobs)
    print(f"[oracle] {len(jobs)} tiles: {wall:.1f} s on {workers} workers", flush=True)
    rows = np.concatenate([oracle.tile_tokens(w.volume, w.tile, t) for t in last])
    for h in range(w.heads):
        assert_close(got[0, h, rows], ref[(0, h)][rows], w.dtype, f"{w.name} head {h} last tiles")


@pytest.mark.parametrize("w", [workloads.STA_18_24_24, workloads.MIXED_HEADS], ids=lambda w: w.name)
def test_full_size_raster_equals_three_call_path(w):
    print(f"[case] full size {w.name}: raster kernel vs reorder path", flush=True)
    inp = workloads.make_inputs(w)
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    a = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows, fused=True)
    b = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_more_than_2_31_elements_per_tensor():
    """B = 4, 48 heads at 30x48x80, d = 128: 2.83e9 elements per tensor, past
    what 32-bit element offsets reach. Rows of the last (batch, head) -- the
    largest offsets -- and of the first are checked against the oracle; the
    raster kernel and the tile-major path agree on the last head."""
    vol, tile, win = (30, 48, 80), (6, 8, 8), (18, 24, 24)
    B, heads, d = 4, 48, 128
    S = vol[0] * vol[1] * vol[2]
    assert B * heads * S * d > 2 ** 31
    print(f"[case] large: B={B} heads={heads} S={S} d={d}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(123)
    shape = (B, heads) + vol + (d,)
    q, k, v = (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
               for _ in range(3))
    out = binding.sta_forward_raster(q, k, v, tile, [win])
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    n = oracle.tile_grid(vol, tile)
    scale = default_scale(d)
    for b, h in ((0, 0), (B - 1, heads - 1)):
        qh, kh, vh = (x[b:b + 1, h:h + 1].float().cpu().numpy() for x in (q, k, v))
        tiles = [0, n[0] * n[1] * n[2] - 1, int(rng.integers(0, n[0] * n[1] * n[2]))]
        rows = np.concatenate([oracle.tile_tokens(vol, tile, t)[rng.choice(384, 8, replace=False)] for t in tiles])
        ref = oracle.sta_attention_rows(qh, kh, vh, tile, win, scale, 0, 0, rows)
        got = out[b, h].float().cpu().numpy().reshape(-1, d)[rows]
        assert_close(got, ref, "bf16", f"large b={b} h={h}")
    # the tile-major path on the last (batch, head) alone gives the same rows,
    # up to rounding: that one-slice problem runs its partly filled last round
    # with each item's key chunks split over two wave groups (a different
    # summation order), which the 57 600 items here, filling every round, do not
    last = [x[B - 1:B, heads - 1:heads].contiguous() for x in (q, k, v)]
    ref_last = binding.sliding_tile_attention(*last, tile, [win], fused=False)
    torch.cuda.synchronize()
    a = ref_last[0, 0].float().cpu().numpy().reshape(-1, d)
    b = out[B - 1, heads - 1].float().cpu().numpy().reshape(-1, d)
    assert_close(a, b.astype(np.float64), "bf16", "large: last slice alone vs in the batch")
    assert (a == b).mean() > 0.5
    del q, k, v, out
    torch.cuda.empty_cache()
