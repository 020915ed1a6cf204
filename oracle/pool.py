"""Process pool over the oracle's (batch, head, query tile) jobs -- TEST
INFRASTRUCTURE.

Only the tests and the benchmark's CPU-baseline leg may import this module. It
holds no attention arithmetic: each job is one call of the oracle's own
``sta_attention_rows`` on the tokens of one query tile, run in a worker
process with one BLAS thread, so that the whole host (its cores as
``os.sched_getaffinity`` reports them, at most ``MAX_WORKERS``) computes
independent tiles side by side.

Workers are forked (no exec): the input arrays are module state set before the
pool starts, shared copy-on-write, never pickled. Nothing in a worker touches
a GPU.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import time
from typing import Iterable, List, Sequence, Tuple

import numpy as np

from .sta_oracle import sta_attention_rows, tile_grid, tile_tokens

# Workers at most: a GPU machine gives one GPU's share of its host, 16 cores,
# whatever the machine reports.
MAX_WORKERS = 16

_STATE = {}


def host_workers() -> int:
    """Cores this process may run on, at most MAX_WORKERS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_WORKERS))


def _one_blas_thread():
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _job(job):
    b, h, tile_index = job
    s = _STATE
    rows = tile_tokens(s["volume"], s["tile"], tile_index)
    window = tuple(int(x) for x in s["windows"][h])
    out = sta_attention_rows(s["q"], s["k"], s["v"], s["tile"], window, s["scale"], b, h, rows)
    return b, h, rows, out


def tile_jobs(volume, tile, pairs: Iterable[Tuple[int, int]], tiles=None) -> List[Tuple[int, int, int]]:
    """(b, h, query tile) jobs for the given (b, h) pairs: every tile, or the
    listed ones."""
    n = tile_grid(volume, tile)
    all_tiles = range(n[0] * n[1] * n[2]) if tiles is None else tiles
    return [(b, h, t) for b, h in pairs for t in all_tiles]


def sta_attention_pool(q, k, v, tile, windows, scale, jobs: Sequence[Tuple[int, int, int]],
                       workers: int | None = None, progress=None):
    """Run the oracle's rows of every job on a process pool.

    q, k, v: (B, heads, T, H, W, d) raster arrays; windows: (heads, 3) tokens.
    Returns ({(b, h): float64 (S, d) array with the rows of the jobs' tiles
    filled, NaN elsewhere}, wall-clock seconds, workers used). `progress`, if
    given, is called with (jobs done, jobs total) as results arrive.
    """
    workers = host_workers() if workers is None else max(1, int(workers))
    volume = tuple(int(x) for x in q.shape[2:5])
    d = q.shape[-1]
    S = volume[0] * volume[1] * volume[2]
    _STATE.clear()
    _STATE.update(q=q, k=k, v=v, tile=tuple(tile), windows=np.asarray(windows).reshape(-1, 3),
                  scale=float(scale), volume=volume)
    out = {}
    for b, h, _ in jobs:
        if (b, h) not in out:
            out[(b, h)] = np.full((S, d), np.nan)
    t0 = time.perf_counter()
    ctx = mp.get_context("fork")
    try:
        with ctx.Pool(workers, initializer=_one_blas_thread) as pool:
            for i, (b, h, rows, res) in enumerate(pool.imap_unordered(_job, jobs, chunksize=1)):
                out[(b, h)][rows] = res
                if progress is not None:
                    progress(i + 1, len(jobs))
    finally:
        _STATE.clear()
    return out, time.perf_counter() - t0, workers
