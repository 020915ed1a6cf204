"""Seeded synthetic workloads for Sliding Tile Attention (STA).

This module only draws and shapes random inputs. It holds none of the
attention arithmetic: no window rule, no tile order, no softmax. Both the HIP
path (through its tests and the benchmark) and the CPU oracle are fed from here,
so that the two sides see identical values.

The pages measure STA on HunyuanVideo activations (a 5 s 720p clip) and on
VBench / MovieGen prompts ("Fast Video Generation with Sliding Tile Attention",
atlas.scime.ai summary, "Experimental setup"). Neither the model nor the
prompts are available, so seeded Gaussian tensors with the same shape stand in
for them: a 30x48x80 latent volume, 24 heads of dimension 128, tile (6,8,8).
The window triples in tokens, (18,24,24), (30,40,40) and the whole volume, are
the ones the same summary lists in its measured-effects table.

Random streams (NumPy PCG64):
  * ``default_rng(seed)``: q, k, v in that order, each
    ``standard_normal((B, heads, T, H, W, d), float32)``;
  * ``default_rng((seed, 1))``: if the windows are drawn, one option index per
    head, ``integers(0, n_options, heads)`` (independent of the tensor sizes, so
    the windows are known without drawing the tensors);
  * ``default_rng((seed, 2))``: if a sinusoid is added, integer frequencies
    ``integers(0, 3, (d, 3))`` (cycles per extent along t, y, x) and phases
    ``uniform(0, 2*pi, d)``; the field
    ``amp * sin(2*pi*(f_t t/T + f_y y/H + f_x x/W) + phase)`` is added to q, k
    and v for every batch entry and head.
Then bf16 workloads are rounded once, round-to-nearest-even, with torch's cast.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

Triple = Tuple[int, int, int]

# Window options for the mixed per-head workload, in tokens (t, h, w).
MIXED_WINDOW_OPTIONS: Tuple[Triple, ...] = (
    (18, 24, 24),
    (18, 40, 40),
    (30, 24, 24),
    (30, 40, 40),
    (30, 48, 80),
)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, tile, per-head windows, dtype and seed of one synthetic case.

    ``windows`` holds one (w_t, w_h, w_w) token triple per head, or is None
    when the windows are drawn from ``window_options`` with the seed.
    """

    name: str
    B: int
    heads: int
    head_dim: int
    volume: Triple  # (T, H, W) latent tokens
    tile: Triple  # (c_t, c_h, c_w) tokens
    windows: Optional[Tuple[Triple, ...]]
    dtype: str  # "f32" or "bf16"
    seed: int
    window_options: Optional[Tuple[Triple, ...]] = None
    sinusoid_amp: float = 0.0

    @property
    def seq_len(self) -> int:
        T, H, W = self.volume
        return T * H * W

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _uniform_windows(heads: int, w: Triple) -> Tuple[Triple, ...]:
    return tuple(tuple(w) for _ in range(heads))


HUNYUAN_VOLUME: Triple = (30, 48, 80)
HUNYUAN_TILE: Triple = (6, 8, 8)

# The five named workloads. Index i+1 is also the seed.
TINY_F32 = Workload(
    name="tiny_f32_12x16x16_w12",
    B=1, heads=2, head_dim=64, volume=(12, 16, 16), tile=(4, 4, 4),
    windows=_uniform_windows(2, (12, 12, 12)), dtype="f32", seed=1,
)
STA_18_24_24 = Workload(
    name="sta_30x48x80_w18x24x24",
    B=1, heads=24, head_dim=128, volume=HUNYUAN_VOLUME, tile=HUNYUAN_TILE,
    windows=_uniform_windows(24, (18, 24, 24)), dtype="bf16", seed=2,
)
STA_30_40_40 = Workload(
    name="sta_30x48x80_w30x40x40",
    B=1, heads=24, head_dim=128, volume=HUNYUAN_VOLUME, tile=HUNYUAN_TILE,
    windows=_uniform_windows(24, (30, 40, 40)), dtype="bf16", seed=3,
)
DENSE_WHOLE = Workload(
    name="sta_30x48x80_whole_volume",
    B=1, heads=24, head_dim=128, volume=HUNYUAN_VOLUME, tile=HUNYUAN_TILE,
    windows=_uniform_windows(24, HUNYUAN_VOLUME), dtype="bf16", seed=4,
)
MIXED_HEADS = Workload(
    name="sta_30x48x80_mixed_heads_sinusoid",
    B=1, heads=24, head_dim=128, volume=HUNYUAN_VOLUME, tile=HUNYUAN_TILE,
    windows=None, dtype="bf16", seed=5,
    window_options=MIXED_WINDOW_OPTIONS, sinusoid_amp=0.5,
)

NAMED: Tuple[Workload, ...] = (TINY_F32, STA_18_24_24, STA_30_40_40, DENSE_WHOLE, MIXED_HEADS)


def by_name(name: str) -> Workload:
    for w in NAMED:
        if w.name == name:
            return w
    raise KeyError(name)


@dataclasses.dataclass
class Inputs:
    """Generated tensors in raster token order, shape (B, heads, T, H, W, d).

    ``q, k, v`` are float32 NumPy arrays holding exactly the values the GPU
    sees (already rounded to bf16 for bf16 workloads). ``windows`` is an int32
    array (heads, 3) of token windows.
    """

    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    windows: np.ndarray


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even) and return them as float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def head_windows(w: Workload) -> np.ndarray:
    """Token windows per head as an int32 (heads, 3) array (drawn if need be)."""
    if w.windows is None:
        if not w.window_options:
            raise ValueError("workload has neither windows nor window options")
        idx = np.random.default_rng((w.seed, 1)).integers(0, len(w.window_options), w.heads)
        return np.asarray([w.window_options[i] for i in idx], dtype=np.int32)
    if len(w.windows) != w.heads:
        raise ValueError("one window triple per head is required")
    return np.asarray(w.windows, dtype=np.int32).reshape(w.heads, 3)


def make_inputs(w: Workload) -> Inputs:
    """Draw q, k, v (and, if asked, windows and a shared sinusoid) for ``w``."""
    rng = np.random.default_rng(w.seed)
    T, H, W = w.volume
    shape = (w.B, w.heads, T, H, W, w.head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    windows = head_windows(w)

    if w.sinusoid_amp:
        d = w.head_dim
        srng = np.random.default_rng((w.seed, 2))
        freq = srng.integers(0, 3, (d, 3))
        phase = srng.uniform(0.0, 2.0 * math.pi, d)
        t = np.arange(T, dtype=np.float64)[:, None, None, None] / T
        y = np.arange(H, dtype=np.float64)[None, :, None, None] / H
        x = np.arange(W, dtype=np.float64)[None, None, :, None] / W
        arg = 2.0 * math.pi * (freq[:, 0] * t + freq[:, 1] * y + freq[:, 2] * x) + phase
        field = (w.sinusoid_amp * np.sin(arg)).astype(np.float32)  # (T, H, W, d)
        q += field
        k += field
        v += field

    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return Inputs(w, q, k, v, windows)


def make_grad_output(w: Workload) -> np.ndarray:
    """The upstream gradient dO for backward tests: N(0,1) of the workload's
    shape from its own stream default_rng((seed, 3)), rounded like the inputs."""
    T, H, W = w.volume
    shape = (w.B, w.heads, T, H, W, w.head_dim)
    g = np.random.default_rng((w.seed, 3)).standard_normal(shape, dtype=np.float32)
    return round_to_bf16(g) if w.dtype == "bf16" else g


def small_case(
    volume: Triple,
    tile: Triple,
    windows: Sequence[Triple],
    head_dim: int = 128,
    B: int = 1,
    dtype: str = "bf16",
    seed: int = 0,
    name: str = "small",
    sinusoid_amp: float = 0.0,
) -> Workload:
    """A free-form workload for parity tests (explicit per-head windows)."""
    return Workload(
        name=name, B=B, heads=len(windows), head_dim=head_dim, volume=tuple(volume),
        tile=tuple(tile), windows=tuple(tuple(x) for x in windows), dtype=dtype,
        seed=seed, sinusoid_amp=sinusoid_amp,
    )
