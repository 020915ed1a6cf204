"""GPU: token permutation and key-tile enumeration, bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_video_tile_amd import binding, workloads
from tests.parity_util import to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize(
    "B,heads,volume,tile,d,dtype",
    [
        (1, 2, (12, 16, 16), (4, 4, 4), 64, "f32"),
        (2, 3, (12, 16, 24), (6, 8, 8), 128, "bf16"),
        (1, 1, (6, 9, 10), (3, 3, 2), 64, "bf16"),
        (1, 2, (5, 7, 3), (1, 7, 1), 32, "f32"),
        (1, 1, (4, 4, 4), (4, 4, 4), 128, "bf16"),  # one tile
        (1, 1, (2, 3, 5), (1, 1, 1), 8, "bf16"),  # one token per tile
    ],
)
def test_reorder_restore_bit_exact(B, heads, volume, tile, d, dtype):
    print(f"[case] reorder B={B} heads={heads} volume={volume} tile={tile} d={d} {dtype}", flush=True)
    rng = np.random.default_rng(123)
    x = rng.standard_normal((B, heads) + volume + (d,), dtype=np.float32)
    xg = to_gpu(x, dtype)
    exact_in = xg.float().cpu().numpy()  # the values the GPU holds
    tm = binding.sta_reorder_tiles(xg, tile)
    expect = oracle.to_tile_major(exact_in, tile)
    assert np.array_equal(tm.float().cpu().numpy(), expect)
    back = binding.sta_restore_order(tm, volume, tile)
    assert torch.equal(back, xg)


def test_reorder_full_size_bit_exact():
    w = workloads.STA_18_24_24
    print(f"[case] reorder full size {w.name}", flush=True)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((w.B, w.heads) + w.volume + (w.head_dim,), dtype=np.float32)
    xg = to_gpu(x, "bf16")
    tm = binding.sta_reorder_tiles(xg, w.tile)
    got = tm.view(torch.int16).cpu().numpy()
    raw = xg.view(torch.int16).cpu().numpy()
    assert np.array_equal(got, oracle.to_tile_major(raw, w.tile))
    back = binding.sta_restore_order(tm, w.volume, w.tile)
    assert torch.equal(back, xg)


@pytest.mark.parametrize("w", workloads.NAMED, ids=lambda w: w.name)
def test_kv_tiles_bit_exact_named(w):
    windows = workloads.head_windows(w)
    print(f"[case] kv_tiles {w.name} windows={windows.tolist()}", flush=True)
    lists, counts = binding.sta_kv_tiles(w.heads, w.volume, w.tile, windows)
    ref_lists, ref_counts = oracle.kv_tile_lists(w.volume, w.tile, windows, max_kv=lists.shape[-1])
    assert np.array_equal(counts.cpu().numpy(), ref_counts)
    assert np.array_equal(lists.cpu().numpy(), ref_lists)


@pytest.mark.parametrize(
    "volume,tile,windows,max_kv",
    [
        ((6, 8, 10), (2, 4, 2), [(4, 8, 6), (2, 4, 2), (6, 8, 10)], None),
        ((8, 8, 8), (2, 2, 2), [(4, 4, 4), (2, 6, 8)], 70),  # even windows, padded rows
        ((4, 4, 4), (4, 4, 4), [(4, 4, 4)], 1),
    ],
)
def test_kv_tiles_bit_exact_small(volume, tile, windows, max_kv):
    print(f"[case] kv_tiles volume={volume} tile={tile} windows={windows}", flush=True)
    windows = np.asarray(windows)
    lists, counts = binding.sta_kv_tiles(len(windows), volume, tile, windows, max_kv=max_kv)
    ref_lists, ref_counts = oracle.kv_tile_lists(volume, tile, windows, max_kv=lists.shape[-1])
    assert np.array_equal(counts.cpu().numpy(), ref_counts)
    assert np.array_equal(lists.cpu().numpy(), ref_lists)
