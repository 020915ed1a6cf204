"""Pins for the CPU oracle: what the pages and the mathematics fix.

None of these tests calls the HIP library. Each compares the oracle with
something other than itself: the pages' printed sparsity, a brute-force window
written from a different definition, closed-form counts, a library softmax
attention, or closed-form outputs of special inputs.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_video_tile_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# An independent window definition (brute force)
# ----------------------------------------------------------------------------

def brute_start(q_tile: int, n: int, omega: int) -> int:
    """The feasible window (start in [0, n - omega]) whose centre is nearest the
    query tile's centre; ties go to the smaller start. Centres in tile units:
    tile q spans [q, q+1), so its centre is q + 1/2; the window spans
    [s, s + omega), centre s + omega/2."""
    best, best_d = None, None
    for s in range(0, n - omega + 1):
        d = abs((s + omega / 2.0) - (q_tile + 0.5))
        if best_d is None or d < best_d - 1e-12:
            best, best_d = s, d
    return best


def brute_token_mask(volume, tile, window):
    """S x S mask from pure-Python loops over every (query, key) token pair."""
    T, H, W = volume
    n = [e // c for e, c in zip(volume, tile)]
    om = [w // c for w, c in zip(window, tile)]
    coords = [(t, y, x) for t in range(T) for y in range(H) for x in range(W)]
    S = len(coords)
    m = np.zeros((S, S), dtype=bool)
    for i, qc in enumerate(coords):
        starts = [brute_start(qc[a] // tile[a], n[a], om[a]) for a in range(3)]
        for j, kc in enumerate(coords):
            m[i, j] = all(starts[a] <= kc[a] // tile[a] < starts[a] + om[a] for a in range(3))
    return m


def sdpa64(q, k, v, scale):
    """Library softmax attention (torch CPU, float64) on (..., S, d) arrays."""
    tq, tk, tv = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()


# ----------------------------------------------------------------------------
# Geometry pins
# ----------------------------------------------------------------------------

def test_pages_sparsity_91_percent_at_18_24_24():
    g = json.load(open(os.path.join(GOLDEN, "pages_sparsity.json")))
    sel = oracle.tile_selection(tuple(g["volume"]), tuple(g["tile"]), tuple(g["window_tokens"]))
    sparsity = 1.0 - sel.sum() / sel.size
    assert round(100 * sparsity) == g["sparsity_percent"]
    # Exactly 1 - 27/300 under the clamped window.
    assert sel.sum() == 27 * 300


def test_truncated_window_would_not_give_the_pages_sparsity():
    """The alternative boundary reading (cut the window at the volume edge)
    gives 93.5%, not the pages' 91%: the pin separates the two readings."""
    n, om = (5, 6, 10), (3, 3, 3)
    pairs = 0
    for q in itertools.product(*[range(x) for x in n]):
        cnt = 1
        for a in range(3):
            lo, hi = max(q[a] - om[a] // 2, 0), min(q[a] - om[a] // 2 + om[a], n[a])
            cnt *= hi - lo
        pairs += cnt
    assert round(100 * (1 - pairs / 90000.0)) == 94


@pytest.mark.parametrize(
    "volume,tile,window",
    [
        ((6, 4, 8), (2, 2, 2), (2, 2, 2)),
        ((6, 4, 8), (2, 2, 2), (6, 4, 6)),
        ((6, 4, 8), (2, 2, 2), (4, 2, 4)),  # even tile counts
        ((6, 6, 6), (3, 2, 1), (3, 4, 3)),
        ((4, 6, 10), (2, 3, 2), (4, 6, 6)),
        ((5, 4, 7), (1, 2, 1), (3, 2, 5)),
    ],
)
def test_token_mask_equals_brute_force(volume, tile, window):
    S = volume[0] * volume[1] * volume[2]
    got = oracle.token_mask_rows(volume, tile, window, np.arange(S))
    assert np.array_equal(got, brute_token_mask(volume, tile, window))


def test_clamp_start_equals_nearest_centre_window_exhaustively():
    for n in range(1, 13):
        for omega in range(1, n + 1):
            for q in range(n):
                assert oracle.window_start(q, n, omega) == brute_start(q, n, omega), (n, omega, q)


def test_axis_selection_closed_forms():
    """Per axis: omega tiles selected, one contiguous interval, own tile inside."""
    for n in range(1, 11):
        for c in (1, 2, 3):
            for omega in range(1, n + 1):
                am = oracle.axis_mask(n * c, c, omega)
                blocks = am.reshape(n, c, n, c)
                sel = blocks.all(axis=(1, 3))
                assert (sel | ~blocks.any(axis=(1, 3))).all()
                for q in range(n):
                    idx = np.nonzero(sel[q])[0]
                    assert len(idx) == omega
                    assert idx[-1] - idx[0] == omega - 1
                    assert idx[0] <= q <= idx[-1]


@pytest.mark.parametrize(
    "window,count,total",
    [
        ((18, 24, 24), 27, 8100),
        ((30, 40, 40), 125, 37500),
        ((30, 48, 80), 300, 90000),
        ((18, 40, 40), 75, 22500),
        ((30, 24, 24), 45, 13500),
    ],
)
def test_hunyuan_shape_counts(window, count, total):
    sel = oracle.tile_selection((30, 48, 80), (6, 8, 8), window)
    assert (sel.sum(axis=1) == count).all()
    assert sel.sum() == total
    assert sel.diagonal().all()  # every window contains its own tile


def test_whole_volume_window_selects_everything():
    sel = oracle.tile_selection((30, 48, 80), (6, 8, 8), (30, 48, 80))
    assert sel.all()


def test_tiny_config_counts():
    w = workloads.TINY_F32
    lists, counts = oracle.kv_tile_lists(w.volume, w.tile, np.asarray(w.windows))
    assert (counts == 27).all()
    assert counts.sum() == 2 * 1296
    assert (np.diff(lists, axis=-1) > 0).all()  # ascending tile order


@pytest.mark.parametrize(
    "volume,tile,window",
    [((12, 16, 16), (4, 4, 4), (12, 12, 12)), ((6, 8, 10), (2, 4, 2), (4, 8, 6)), ((8, 8, 8), (2, 2, 2), (2, 6, 4))],
)
def test_tile_selection_equals_token_mask_blocks(volume, tile, window):
    a = oracle.tile_selection(volume, tile, window)
    b = oracle.tile_selection_from_token_mask(volume, tile, window)
    assert np.array_equal(a, b)


def test_token_wise_window_would_make_mixed_blocks(monkeypatch):
    """Plant the token-wise sliding window (the design STA replaces) in the
    oracle: the no-mixed-block check must fire."""

    def token_wise_axis_mask(extent, c, omega):
        r = np.arange(extent)
        half = omega * c // 2
        start = np.clip(r - half, 0, extent - omega * c)
        return (r[None, :] >= start[:, None]) & (r[None, :] < start[:, None] + omega * c)

    monkeypatch.setattr(oracle.sta_oracle, "axis_mask", token_wise_axis_mask)
    with pytest.raises(AssertionError, match="mixed block"):
        oracle.sta_oracle.tile_selection((12, 16, 16), (4, 4, 4), (4, 8, 8))


def test_kv_pair_count():
    assert oracle.kv_pair_count((30, 48, 80), (6, 8, 8), np.array([[18, 24, 24], [30, 48, 80]])) == 8100 + 90000


def test_invalid_geometry_rejected():
    with pytest.raises(ValueError):
        oracle.tile_grid((30, 48, 80), (0, 8, 8))
    with pytest.raises(ValueError):
        oracle.window_in_tiles((20, 24, 24), (6, 8, 8), (30, 48, 80))
    with pytest.raises(ValueError):
        oracle.window_in_tiles((36, 24, 24), (6, 8, 8), (30, 48, 80))
    # a tile that does not divide the volume covers it with a padded grid
    assert oracle.tile_grid((30, 48, 80), (7, 8, 8)) == (5, 6, 10)
    assert oracle.window_in_tiles((35, 24, 24), (7, 8, 8), (30, 48, 80)) == (5, 3, 3)


# ----------------------------------------------------------------------------
# Token order pins
# ----------------------------------------------------------------------------

def test_tile_major_order_brute_force():
    rng = np.random.default_rng(0)
    volume, tile = (4, 6, 4), (2, 3, 2)
    T, H, W = volume
    x = rng.standard_normal((2, 3, T, H, W, 5))
    y = oracle.to_tile_major(x, tile)
    nt, nh, nw = T // 2, H // 3, W // 2
    expect = np.empty_like(y)
    pos = 0
    for it in range(nt):
        for ih in range(nh):
            for iw in range(nw):
                for lt in range(2):
                    for lh in range(3):
                        for lw in range(2):
                            expect[:, :, pos] = x[:, :, it * 2 + lt, ih * 3 + lh, iw * 2 + lw]
                            pos += 1
    assert np.array_equal(y, expect)
    assert np.array_equal(oracle.from_tile_major(y, volume, tile), x)


def test_tile_tokens_matches_tile_major_order():
    volume, tile = (6, 8, 8), (2, 4, 4)
    S = 6 * 8 * 8
    ids = np.arange(S, dtype=np.float64).reshape(1, 1, 6, 8, 8, 1)
    tm = oracle.to_tile_major(ids, tile).reshape(-1).astype(int)
    tau = 32
    for j in range(S // tau):
        assert np.array_equal(tm[j * tau:(j + 1) * tau], oracle.tile_tokens(volume, tile, j))


# ----------------------------------------------------------------------------
# Output pins
# ----------------------------------------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_whole_volume_window_equals_library_attention():
    volume, tile, d = (4, 8, 8), (2, 4, 4), 16
    q, k, v = (_rand((1, 2) + volume + (d,), s) for s in (1, 2, 3))
    scale = 1 / math.sqrt(d)
    got = oracle.sta_attention(q, k, v, tile, np.array([volume, volume]), scale)
    S = 4 * 8 * 8
    ref = sdpa64(q.reshape(1, 2, S, d), k.reshape(1, 2, S, d), v.reshape(1, 2, S, d), scale)
    np.testing.assert_allclose(got.reshape(1, 2, S, d), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.full_attention(q, k, v, scale).reshape(1, 2, S, d), ref,
                               rtol=1e-12, atol=1e-12)


def test_single_tile_window_is_per_tile_attention():
    volume, tile, d = (4, 4, 6), (2, 2, 3), 8
    q, k, v = (_rand((1, 1) + volume + (d,), s) for s in (4, 5, 6))
    scale = 0.3
    got = oracle.sta_attention(q, k, v, tile, np.array([tile]), scale)
    for t0 in range(0, 4, 2):
        for y0 in range(0, 4, 2):
            for x0 in range(0, 6, 3):
                sl = (0, 0, slice(t0, t0 + 2), slice(y0, y0 + 2), slice(x0, x0 + 3))
                ref = sdpa64(q[sl].reshape(-1, d), k[sl].reshape(-1, d), v[sl].reshape(-1, d), scale)
                np.testing.assert_allclose(got[sl].reshape(-1, d), ref, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_window_values():
    volume, tile, d = (6, 8, 8), (2, 2, 2), 4
    window = (2, 6, 4)
    v = _rand((1, 1) + volume + (d,), 7)
    q = np.zeros_like(v)
    k = _rand(v.shape, 8)
    got = oracle.sta_attention(q, k, v, tile, np.array([window]), 1.0)
    n = [e // c for e, c in zip(volume, tile)]
    om = [w // c for w, c in zip(window, tile)]
    for t in range(6):
        for y in range(8):
            for x in range(8):
                s = [brute_start(c // tc, nn, o) for c, tc, nn, o in zip((t, y, x), tile, n, om)]
                box = v[0, 0,
                        s[0] * tile[0]:(s[0] + om[0]) * tile[0],
                        s[1] * tile[1]:(s[1] + om[1]) * tile[1],
                        s[2] * tile[2]:(s[2] + om[2]) * tile[2]]
                np.testing.assert_allclose(got[0, 0, t, y, x], box.reshape(-1, d).mean(axis=0),
                                           rtol=1e-12, atol=1e-12)


def test_constant_values_give_constant_output():
    volume, tile, d = (4, 4, 4), (2, 2, 2), 6
    q, k = _rand((1, 1) + volume + (d,), 9), _rand((1, 1) + volume + (d,), 10)
    const = np.arange(d, dtype=np.float64) - 2.5
    v = np.broadcast_to(const, q.shape).copy()
    got = oracle.sta_attention(q, k, v, tile, np.array([(2, 2, 4)]), 0.5)
    np.testing.assert_allclose(got, np.broadcast_to(const, got.shape), rtol=1e-13, atol=1e-13)


def test_large_logits_stay_finite():
    volume, tile, d = (2, 2, 4), (1, 2, 2), 4
    q, k, v = (_rand((1, 1) + volume + (d,), s) for s in (11, 12, 13))
    got = oracle.sta_attention(q * 1e3, k * 1e3, v, tile, np.array([(2, 2, 2)]), 1.0)
    assert np.isfinite(got).all()


def test_rows_match_full_output():
    """The row-subset entry point (used by the sampled full-size checks) picks
    the right batch entry, head and window: it equals the matching rows of the
    whole output for every (b, h) of a B = 2, three-head draw with a different
    window per head."""
    w = workloads.small_case((6, 8, 12), (2, 4, 4), [(2, 4, 4), (6, 8, 12), (4, 4, 8)],
                             head_dim=16, dtype="f32", B=2, seed=5, name="rows")
    inp = workloads.make_inputs(w)
    scale = 1 / math.sqrt(w.head_dim)
    full = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, scale)
    rows = np.array([0, 17, 300, 575])
    for b in range(w.B):
        for h in range(w.heads):
            part = oracle.sta_attention_rows(inp.q, inp.k, inp.v, w.tile, tuple(inp.windows[h]),
                                             scale, b, h, rows)
            np.testing.assert_allclose(part, full[b, h].reshape(-1, w.head_dim)[rows],
                                       rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize(
    "volume,tile,windows",
    [
        # the pages' geometry, with the other named windows and an even one
        ((30, 48, 80), (6, 8, 8), [(18, 24, 24), (30, 40, 40), (30, 24, 24), (12, 16, 16)]),
        ((12, 16, 16), (4, 4, 4), [(12, 12, 12), (4, 8, 4)]),
        # a padded tile grid (the volume is not whole tiles)
        ((5, 6, 7), (2, 4, 4), [(4, 4, 4), (2, 8, 8), (6, 8, 8)]),
        ((11, 9, 13), (4, 4, 12), [(8, 8, 12), (12, 12, 24)]),
    ],
)
def test_kv_tile_lists_equal_brute_force_listing(volume, tile, windows):
    """List contents, not only their counts: per head and query tile, the key
    tiles of the nearest-centre window (brute_start, a definition independent
    of the oracle's clamp) enumerated by nested loops in raster order of tile
    coordinates, then -1 fill. A listing taken from the wrong axis of the
    selection (the transposed relation, which differs under clamping) fails."""
    lists, counts = oracle.kv_tile_lists(volume, tile, np.array(windows))
    n = [-(-e // c) for e, c in zip(volume, tile)]
    assert lists.shape[:2] == (len(windows), n[0] * n[1] * n[2])
    for h, win in enumerate(windows):
        om = [win[a] // tile[a] for a in range(3)]
        for i, qc in enumerate(itertools.product(range(n[0]), range(n[1]), range(n[2]))):
            st = [brute_start(qc[a], n[a], om[a]) for a in range(3)]
            want = [(t * n[1] + y) * n[2] + x
                    for t in range(st[0], st[0] + om[0])
                    for y in range(st[1], st[1] + om[1])
                    for x in range(st[2], st[2] + om[2])]
            assert counts[h, i] == len(want), (h, i)
            assert list(lists[h, i, :counts[h, i]]) == want, (h, i)
            assert (lists[h, i, counts[h, i]:] == -1).all()
