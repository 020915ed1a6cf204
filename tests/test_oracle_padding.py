"""Pins for the oracle on volumes the tile does not divide (padded tile grid).

The grid has ceil(extent / c) tiles per axis; windows follow the same clamp
rule on that grid; padded positions are neither keys nor queries. Each test
compares the oracle with something other than itself: a brute-force window
from a different definition, library attention and its gradient, index loops
for the padded tile-major layout, and closed forms.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle import brute_start

PADDED = [
    ((5, 6, 7), (2, 4, 4), (4, 4, 4)),
    ((5, 6, 7), (2, 4, 4), (2, 8, 8)),
    ((3, 5, 9), (2, 2, 4), (2, 4, 8)),
    ((7, 3, 5), (3, 2, 2), (6, 2, 4)),
]


def brute_padded_mask(volume, tile, window):
    """Token mask by loops: tile grid of ceil(extent / c), nearest-centre window."""
    T, H, W = volume
    n = [-(-e // c) for e, c in zip(volume, tile)]
    om = [w // c for w, c in zip(window, tile)]
    coords = [(t, y, x) for t in range(T) for y in range(H) for x in range(W)]
    m = np.zeros((len(coords), len(coords)), dtype=bool)
    for i, qc in enumerate(coords):
        st = [brute_start(qc[a] // tile[a], n[a], om[a]) for a in range(3)]
        for j, kc in enumerate(coords):
            m[i, j] = all(st[a] <= kc[a] // tile[a] < st[a] + om[a] for a in range(3))
    return m


@pytest.mark.parametrize("volume,tile,window", PADDED)
def test_padded_token_mask_equals_brute_force(volume, tile, window):
    S = volume[0] * volume[1] * volume[2]
    got = oracle.token_mask_rows(volume, tile, window, np.arange(S))
    assert np.array_equal(got, brute_padded_mask(volume, tile, window))


@pytest.mark.parametrize("volume,tile,window", PADDED)
def test_padded_tile_selection_counts(volume, tile, window):
    """Every query tile of the padded grid selects prod(omega) key tiles; the
    transposed lists total the same."""
    n = oracle.tile_grid(volume, tile)
    om = oracle.window_in_tiles(window, tile, volume)
    sel = oracle.tile_selection(volume, tile, window)
    assert sel.shape == (n[0] * n[1] * n[2],) * 2
    assert (sel.sum(axis=1) == om[0] * om[1] * om[2]).all()
    _, counts = oracle.q_tile_lists(volume, tile, [window])
    assert counts.sum() == sel.sum()


def test_padded_tile_tokens_cover_the_volume_once():
    volume, tile = (5, 6, 7), (2, 4, 4)
    n = oracle.tile_grid(volume, tile)
    toks = np.concatenate([oracle.tile_tokens(volume, tile, i) for i in range(n[0] * n[1] * n[2])])
    assert np.array_equal(np.sort(toks), np.arange(5 * 6 * 7))


def test_padded_tile_major_layout_by_loops():
    volume, tile = (3, 5, 6), (2, 2, 4)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 2) + volume + (4,))
    y = oracle.to_tile_major(x, tile)
    n = oracle.tile_grid(volume, tile)
    tau = tile[0] * tile[1] * tile[2]
    assert y.shape == (1, 2, n[0] * n[1] * n[2] * tau, 4)
    for it in range(n[0]):
        for ih in range(n[1]):
            for iw in range(n[2]):
                tidx = (it * n[1] + ih) * n[2] + iw
                for lt in range(tile[0]):
                    for lh in range(tile[1]):
                        for lw in range(tile[2]):
                            row = tidx * tau + (lt * tile[1] + lh) * tile[2] + lw
                            t, yy, xx = it * tile[0] + lt, ih * tile[1] + lh, iw * tile[2] + lw
                            if t < volume[0] and yy < volume[1] and xx < volume[2]:
                                assert np.array_equal(y[:, :, row], x[:, :, t, yy, xx])
                            else:
                                assert not y[:, :, row].any()
    assert np.array_equal(oracle.from_tile_major(y, volume, tile), x)


def sdpa64(q, k, v, scale):
    tq, tk, tv = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()


def test_padded_whole_grid_window_is_full_attention():
    volume, tile = (5, 6, 7), (2, 4, 4)
    n = oracle.tile_grid(volume, tile)
    whole = tuple(na * c for na, c in zip(n, tile))   # (6, 8, 8): the whole padded grid
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 2) + volume + (8,)) for _ in range(3))
    got = oracle.sta_attention(q, k, v, tile, [whole, whole], 0.3)
    ref = sdpa64(q.reshape(1, 2, -1, 8), k.reshape(1, 2, -1, 8), v.reshape(1, 2, -1, 8), 0.3)
    np.testing.assert_allclose(got.reshape(ref.shape), ref, rtol=1e-11, atol=1e-12)


def test_padded_single_tile_window_is_per_tile_attention():
    volume, tile = (5, 6, 7), (2, 4, 4)
    n = oracle.tile_grid(volume, tile)
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 1) + volume + (8,)) for _ in range(3))
    got = oracle.sta_attention(q, k, v, tile, [tile], 0.4).reshape(-1, 8)
    qf, kf, vf = (a.reshape(-1, 8) for a in (q, k, v))
    for i in range(n[0] * n[1] * n[2]):
        toks = oracle.tile_tokens(volume, tile, i)   # real tokens of the tile only
        ref = sdpa64(qf[toks], kf[toks], vf[toks], 0.4)
        np.testing.assert_allclose(got[toks], ref, rtol=1e-11, atol=1e-12)


def test_padded_zero_query_gives_window_mean():
    volume, tile, window = (5, 6, 7), (2, 4, 4), (4, 4, 4)
    rng = np.random.default_rng(6)
    k, v = (rng.standard_normal((1, 1) + volume + (8,)) for _ in range(2))
    q = np.zeros_like(k)
    got = oracle.sta_attention(q, k, v, tile, [window], 1.0)[0, 0]
    n = oracle.tile_grid(volume, tile)
    om = [w // c for w, c in zip(window, tile)]
    for t in range(volume[0]):
        for y in range(volume[1]):
            for x in range(volume[2]):
                st = [brute_start(c // tl, na, o) for c, tl, na, o in zip((t, y, x), tile, n, om)]
                sl = [slice(s * tl, min((s + o) * tl, e)) for s, tl, o, e in zip(st, tile, om, volume)]
                want = v[0, 0, sl[0], sl[1], sl[2]].reshape(-1, 8).mean(axis=0)
                np.testing.assert_allclose(got[t, y, x], want, rtol=1e-12, atol=1e-13)


def test_padded_gradients_match_central_differences():
    volume, tile, windows = (3, 5, 6), (2, 2, 4), [(2, 4, 4), (4, 6, 8)]
    rng = np.random.default_rng(8)
    shape = (1, 2) + volume + (8,)
    q, k, v, dout = (rng.standard_normal(shape) for _ in range(4))
    dq, dk, dv = oracle.sta_backward(q, k, v, dout, tile, windows, 0.45)
    eps = 1e-5
    pick = np.random.default_rng(9)

    def loss(a, b, c):
        return float(np.sum(dout * oracle.sta_attention(a, b, c, tile, windows, 0.45)))

    for which, g in ((0, dq), (1, dk), (2, dv)):
        for _ in range(25):
            idx = tuple(int(pick.integers(0, s)) for s in shape)
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 + 1e-6 * abs(fd)
