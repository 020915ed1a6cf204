"""GPU: STA forward and the dense comparator against the float64 oracle,
element by element, on small seeded workloads that span several tiles."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_video_tile_amd import binding, workloads
from tests.parity_util import assert_close, default_scale, to_gpu

pytestmark = pytest.mark.gpu


def run_sta(inp: workloads.Inputs, scale=None, fused=True):
    """The whole path on raster inputs -> numpy. fused: the one raster-order
    kernel; else reorder -> tile-major forward -> restore."""
    w = inp.workload
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    out = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows, scale, fused=fused)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


SMALL_CASES = [
    # name, volume, tile, windows per head, head_dim, dtype
    ("hunyuan_tiles_2x2x3", (12, 16, 24), (6, 8, 8), [(6, 8, 8), (12, 16, 24), (6, 16, 8)], 128, "bf16"),
    ("tile64_3x4x4_w333", (12, 16, 16), (4, 4, 4), [(12, 12, 12), (4, 4, 4)], 128, "bf16"),
    ("tile64_d64", (12, 16, 16), (4, 4, 4), [(12, 12, 12), (8, 8, 8)], 64, "bf16"),  # even windows
    ("tile48_ragged_runs", (9, 8, 12), (3, 4, 4), [(6, 4, 8), (9, 8, 12)], 128, "bf16"),
    ("tile128", (8, 8, 16), (4, 4, 8), [(4, 8, 8), (8, 4, 16)], 128, "bf16"),
    ("tile8_tiny", (4, 4, 6), (2, 2, 2), [(2, 2, 2), (4, 4, 6), (4, 2, 4)], 128, "bf16"),
    ("one_tile_volume", (6, 8, 8), (6, 8, 8), [(6, 8, 8)], 128, "bf16"),
    # 2D (image) STA: one frame, tiles of 1 x 8 x 8 (a 2D window slid tile by tile)
    ("image_2d_tile8x8", (1, 32, 48), (1, 8, 8), [(1, 24, 24), (1, 32, 48), (1, 8, 16)], 128, "bf16"),
    ("f32_tiny_like", (12, 16, 16), (4, 4, 4), [(12, 12, 12), (4, 8, 12)], 64, "f32"),
    ("f32_d128", (6, 8, 8), (2, 4, 4), [(4, 8, 4), (6, 8, 8)], 128, "f32"),
    ("f32_ragged", (9, 8, 12), (3, 4, 4), [(6, 4, 8)], 64, "f32"),
]


@pytest.mark.parametrize("fused", [True, False], ids=["raster", "tile_major"])
@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: c[0])
def test_forward_matches_oracle(case, fused):
    name, volume, tile, windows, d, dtype = case
    w = workloads.small_case(volume, tile, windows, head_dim=d, dtype=dtype, seed=11, name=name)
    print(f"[case] forward fused={fused} {w}", flush=True)
    inp = workloads.make_inputs(w)
    got = run_sta(inp, fused=fused)
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, tile, inp.windows, default_scale(d))
    assert_close(got, ref, dtype, name)


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: c[0])
def test_raster_kernel_equals_three_call_path(case):
    """The raster-order kernel does the same arithmetic in the same order as
    reorder + tile-major forward + restore, so the outputs agree bit for bit."""
    name, volume, tile, windows, d, dtype = case
    w = workloads.small_case(volume, tile, windows, head_dim=d, dtype=dtype, B=2, seed=12, name=name)
    print(f"[case] raster vs tile-major {w}", flush=True)
    inp = workloads.make_inputs(w)
    a = run_sta(inp, fused=True)
    b = run_sta(inp, fused=False)
    assert np.array_equal(a, b), f"{name}: max diff {np.abs(a - b).max()}"


def test_raster_run_limit():
    """A window run longer than the raster kernel's offset table (8192 keys) is
    refused by sta_forward_raster; sliding_tile_attention then takes the
    reorder path."""
    w = workloads.small_case((1, 1, 8200), (1, 1, 8), [(1, 1, 8200)], head_dim=64, seed=13,
                             name="run_8200")
    print(f"[case] raster limit {w}", flush=True)
    inp = workloads.make_inputs(w)
    q, k, v = (to_gpu(x, "bf16") for x in (inp.q, inp.k, inp.v))
    with pytest.raises(NotImplementedError):
        binding.sta_forward_raster(q, k, v, w.tile, inp.windows)
    got = run_sta(inp)
    # The window spans the whole volume, so STA is full attention here.
    ref = oracle.full_attention(inp.q, inp.k, inp.v, default_scale(64)).reshape(got.shape)
    assert_close(got, ref, "bf16", w.name)


def test_forward_batch_and_sinusoid():
    w = workloads.small_case((12, 16, 24), (6, 8, 8), [(6, 16, 8), (12, 8, 24)], B=2, seed=5,
                             sinusoid_amp=0.5, name="batch2_sinusoid")
    print(f"[case] forward {w}", flush=True)
    inp = workloads.make_inputs(w)
    got = run_sta(inp, scale=0.2)
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, 0.2)
    assert_close(got, ref, "bf16", w.name)


def test_tiny_named_config():
    w = workloads.TINY_F32
    print(f"[case] forward {w.name}", flush=True)
    inp = workloads.make_inputs(w)
    got = run_sta(inp)
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, default_scale(w.head_dim))
    assert_close(got, ref, "f32", w.name)


def test_zero_query_gives_window_mean():
    w = workloads.small_case((12, 16, 24), (6, 8, 8), [(6, 8, 24)], seed=3, name="zero_q")
    print(f"[case] forward {w.name}", flush=True)
    inp = workloads.make_inputs(w)
    inp.q[...] = 0.0
    got = run_sta(inp)
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, 1.0)
    assert_close(got, ref, "bf16", w.name)


def test_constant_values_pass_through():
    w = workloads.small_case((12, 16, 16), (4, 4, 4), [(8, 8, 8)], seed=4, name="const_v")
    print(f"[case] forward {w.name}", flush=True)
    inp = workloads.make_inputs(w)
    const = workloads.round_to_bf16(np.linspace(-2, 2, w.head_dim, dtype=np.float32))
    inp.v[...] = const
    got = run_sta(inp)
    np.testing.assert_allclose(got, np.broadcast_to(const, got.shape), rtol=0, atol=2e-2)


def test_forward_is_deterministic():
    w = workloads.small_case((12, 16, 24), (6, 8, 8), [(6, 16, 8)], seed=8, name="det")
    print(f"[case] forward determinism {w.name}", flush=True)
    inp = workloads.make_inputs(w)
    a, b = run_sta(inp), run_sta(inp)
    assert np.array_equal(a, b)


def test_whole_volume_window_equals_dense_kernel():
    w = workloads.small_case((12, 16, 24), (6, 8, 8), [(12, 16, 24), (12, 16, 24)], seed=9, name="whole")
    print(f"[case] whole-volume STA vs dense kernel", flush=True)
    inp = workloads.make_inputs(w)
    sta = run_sta(inp)
    q, k, v = (to_gpu(x.reshape(w.B, w.heads, -1, w.head_dim), "bf16") for x in (inp.q, inp.k, inp.v))
    dense = binding.sta_full_attention(q, k, v).float().cpu().numpy().reshape(sta.shape)
    ref = oracle.full_attention(inp.q, inp.k, inp.v, default_scale(w.head_dim))
    assert_close(sta, ref, "bf16", "whole-volume STA")
    assert_close(dense, ref, "bf16", "dense kernel")
    assert np.abs(sta - dense).max() <= 2e-2


@pytest.mark.parametrize("S,d,dtype", [(1, 128, "bf16"), (100, 128, "bf16"), (1000, 64, "bf16"),
                                       (4608, 128, "bf16"), (777, 64, "f32"), (300, 128, "f32")])
def test_dense_kernel_matches_oracle(S, d, dtype):
    print(f"[case] dense S={S} d={d} {dtype}", flush=True)
    rng = np.random.default_rng(S + d)
    shape = (1, 2, S, d)
    xs = [rng.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    if dtype == "bf16":
        xs = [workloads.round_to_bf16(x) for x in xs]
    q, k, v = (to_gpu(x, dtype) for x in xs)
    got = binding.sta_full_attention(q, k, v).float().cpu().numpy()
    ref = oracle.full_attention(*xs, default_scale(d))
    assert_close(got, ref, dtype, f"dense S={S}")


def test_large_logits_are_stable():
    w = workloads.small_case((12, 16, 16), (4, 4, 4), [(8, 8, 8)], seed=6, name="large_logits")
    print(f"[case] forward {w.name}", flush=True)
    inp = workloads.make_inputs(w)
    inp.q *= 8.0
    inp.q = workloads.round_to_bf16(inp.q)
    got = run_sta(inp)
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, default_scale(w.head_dim))
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", w.name)


def _tile_grid(volume, tile):
    """Tile coordinates (t, h, w) of every raster token, each (T, H, W)."""
    t, h, w = np.meshgrid(*(np.arange(n) // c for n, c in zip(volume, tile)), indexing="ij")
    return t, h, w


@pytest.mark.parametrize("fused", [True, False], ids=["raster", "tile_major"])
def test_key_scales_jumping_between_tiles(fused):
    """Key magnitudes that change by up to 13x from tile to tile: scores jump
    by orders of magnitude (in log2 units, far past the lazy bound of 8) in the
    middle of every window walk, in both directions. Every chunk is full, so
    the walk takes the path whose reference max moves only when a lane's
    chunk sum exceeds 2^8."""
    w = workloads.small_case((12, 16, 16), (4, 4, 4), [(8, 8, 8), (12, 16, 16)], seed=17,
                             name="key_scale_jumps")
    print(f"[case] forward {w.name} fused={fused}", flush=True)
    inp = workloads.make_inputs(w)
    t, h, x = _tile_grid(w.volume, w.tile)
    factor = 1.0 + 3.0 * ((t * 7 + h * 3 + x) % 5)
    inp.k = workloads.round_to_bf16(inp.k * factor[None, None, :, :, :, None])
    got = run_sta(inp, fused=fused)
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, default_scale(w.head_dim))
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", w.name)


@pytest.mark.parametrize("fused", [True, False], ids=["raster", "tile_major"])
def test_many_moderate_scores_move_the_reference_max(fused):
    """Half the key tiles score about 5 (log2 units) above the others: a
    chunk of them gives probabilities near 2^5 against a max set by the low
    tiles, far below the single-probability bound 2^8, but lane sums of 16
    such probabilities pass 2^8, so the rescale must be triggered by the sum."""
    d = 128
    w = workloads.small_case((8, 16, 16), (4, 4, 4), [(8, 8, 12)], head_dim=d, seed=23,
                             name="moderate_scores")
    print(f"[case] forward {w.name} fused={fused}", flush=True)
    inp = workloads.make_inputs(w)
    scale = default_scale(d)
    alpha = 5.0 / (scale * math.log2(math.e))
    e0 = np.zeros(d, dtype=np.float32)
    e0[0] = 1.0
    t, h, x = _tile_grid(w.volume, w.tile)
    high = ((t + h + x) % 2).astype(np.float32)
    inp.q = workloads.round_to_bf16(alpha * e0 + 0.05 * inp.q)
    inp.k = workloads.round_to_bf16(high[None, None, :, :, :, None] * e0 + 0.05 * inp.k)
    got = run_sta(inp, scale, fused=fused)
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, scale)
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", w.name)


def test_invalid_inputs_raise_before_launch():
    q = torch.zeros((1, 1, 384, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        binding.sta_forward(q, q.clone(), q.clone(), (6, 8, 8), (6, 8, 8), [(7, 8, 8)])
    with pytest.raises(NotImplementedError):
        x = torch.zeros((1, 1, 384, 96), dtype=torch.bfloat16, device="cuda")
        binding.sta_forward(x, x.clone(), x.clone(), (6, 8, 8), (6, 8, 8), [(6, 8, 8)])
    with pytest.raises(TypeError):
        x = torch.zeros((1, 1, 384, 128), dtype=torch.float16, device="cuda")
        binding.sta_forward(x, x.clone(), x.clone(), (6, 8, 8), (6, 8, 8), [(6, 8, 8)])
    r = torch.zeros((1, 1, 6, 8, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        binding.sta_forward_raster(r, r.clone(), r.clone(), (6, 8, 8), [(6, 8, 16)])
    with pytest.raises(ValueError):
        binding.sta_forward_raster(r, r.clone(), r, (6, 8, 8), [(6, 8, 8)], out=r)
